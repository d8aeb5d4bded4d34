/*
 * fq.h -- C ABI of the grouped-expert fake-quant library for AMD MI355X (gfx950).
 *
 * Scale-only quantisation-aware training of a MoE expert layer: the BF16 expert
 * weights stay frozen, weights and every matmul input are fake-quantised
 * (quantised, then dequantised) and only the quantiser scales receive
 * gradients (AngelSlim "MCoreQAD Backend" page, opening paragraph; nxmr.cn
 * article on the same backend, sections 一 and 二.3).  The experts of a layer
 * are 3D-stacked, fake-quantised in one pass and multiplied by one grouped GEMM
 * (nxmr.cn article, section 二.4).  The formats are those of the support matrix
 * (AngelSlim page, Support Matrix; nxmr.cn article, section 三).
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device pointers; "host" pointers are
 *     read before the call returns.  The caller owns every buffer; the library
 *     allocates nothing and keeps no state between calls (one exception:
 *     fq_scale_adamw_noalloc's fixed scratch array, described there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All device work is enqueued on it asynchronously; nothing is synchronised
 *     and nothing is read back to the host.
 *   - Every call returns an fq_status.  Arguments are validated on the host
 *     before any HIP call; on a validation error nothing is launched.
 *   - A saved or workspace buffer belongs to one call at a time: calls that
 *     share one must be ordered (same stream, or synchronised).
 *   - Gradients are overwritten, never accumulated.  Results are bitwise
 *     deterministic for fixed inputs (no floating-point atomics).
 *   - Device data are not checked: routing ids must lie in [0, E) and be
 *     distinct per token, scales must be finite and > 0, inputs finite.
 *     Violations give unspecified values (but no out-of-bounds access:
 *     ids are range-checked by the kernels that index with them).
 *   - bf16 tensors are row-major, 16-byte aligned; fp32 tensors 4-byte aligned.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status --------------------------------------------------------------- */
typedef enum {
    FQ_OK = 0,
    FQ_E_INVALID = -1,      /* null pointer, bad enum, inconsistent request    */
    FQ_E_SHAPE = -2,        /* size negative or not divisible as required      */
    FQ_E_UNSUPPORTED = -3,  /* valid descriptor this library does not implement */
    FQ_E_WORKSPACE = -4,    /* workspace / saved buffer smaller than required  */
    FQ_E_ALIGN = -5,        /* pointer not aligned as required                 */
    FQ_E_HIP = -6           /* a HIP runtime call failed: see fq_last_hip_error */
} fq_status;

/* ---- quantiser descriptor ------------------------------------------------- */
typedef enum {
    FQ_NONE = 0,       /* quantiser disabled: identity (the BF16 teacher path)   */
    FQ_NVFP4 = 1,      /* E2M1 elements, E4M3 block factor per 16, fp32 tensor scale */
    FQ_INT = 2,        /* two's-complement integer grid [qmin, qmax]              */
    FQ_FP8E4M3 = 3     /* OCP E4M3FN (max 448, saturating)                        */
} fq_kind;

typedef enum {
    FQ_PER_TENSOR = 0, /* one scale per matrix (per batch entry / per expert)    */
    FQ_PER_ROW = 1,    /* one scale per row: output channel (W) or token (A)     */
    FQ_PER_GROUP = 2   /* one scale per `group` consecutive elements of a row    */
} fq_gran;

typedef enum {
    FQ_LEARNABLE = 0,  /* scale is a trainable input; its gradient can be formed */
    FQ_STATIC = 1,     /* calibrated scale, no gradient                          */
    FQ_DYNAMIC = 2     /* scale = amax / max-code computed on the fly, detached  */
} fq_source;

typedef struct {
    int32_t kind;      /* fq_kind                                                */
    int32_t gran;      /* fq_gran                                                */
    int32_t group;     /* FQ_PER_GROUP: elements per scale (16 for NVFP4)        */
    int32_t source;    /* fq_source                                              */
    int32_t qmin;      /* FQ_INT only: e.g. -8 / 7 (INT4), -128 / 127 (INT8)     */
    int32_t qmax;
} fq_qdesc;

/*
 * Numbers of one quantiser (every step is one IEEE fp32 operation):
 *   effective scale s^ per element:
 *     NVFP4, learnable/static:  d = E4M3(s_b / t), s^ = t * d   (s_b per 16-block, t per matrix)
 *     NVFP4, dynamic:           d = E4M3(amax_16 / (6 t)), s^ = t * d   (t learnable)
 *     INT/FP8, learnable/static: s^ = scale[tensor | row | group]
 *     INT/FP8, dynamic:          s^ = amax(row | group) / (qmax | 448)
 *   r = x / s^ (correctly rounded), q = nearest grid value of clamp(r), ties to
 *   the even code, y = bf16_rne(q * s^).  s^ == 0 gives q = +-0, y = +-0.
 *   Straight-through backward: dL/dx = g * [qmin <= r <= qmax] (learnable, static)
 *   or g (dynamic); dL/ds = sum g * c, c = q - r inside, qmin/qmax outside;
 *   for NVFP4 the learnable tensor scale of a dynamic quantiser gets sum g * c * d.
 * Codes: NVFP4 nibble = sign(x) << 3 | E2M1 magnitude code; INT two's complement;
 * FP8 byte = sign(x) << 7 | E4M3 magnitude code.  4-bit codes pack two per byte,
 * the even column in the low nibble.  NVFP4 block-scale code = E4M3 byte of d.
 */

/* ---- format presets (the six names of the support matrix) ----------------- */
typedef enum {
    FQ_FMT_NVFP4 = 0,     /* W: NVFP4 learnable block scales; A: NVFP4 dynamic blocks, learnable tensor scale */
    FQ_FMT_NVFP4A16 = 1,  /* W: NVFP4; A: bf16                                   */
    FQ_FMT_W4A16 = 2,     /* W: INT4 [-8,7] learnable per group of 128; A: bf16  */
    FQ_FMT_W8A8 = 3,      /* W: INT8 learnable per output channel; A: INT8 dynamic per token */
    FQ_FMT_FP8 = 4,       /* W: FP8 learnable per output channel; A: FP8 dynamic per token */
    FQ_FMT_W4AFP8 = 5     /* W: INT4 per group of 128; A: FP8 learnable per-expert tensor scale */
} fq_format;

/* Fill the four quantiser descriptors (host pointers) of a format.
 * Errors: FQ_E_INVALID for a null pointer or an unknown format. */
int fq_preset(int32_t format, fq_qdesc* w1, fq_qdesc* w2, fq_qdesc* a1, fq_qdesc* a2);

/* ---- one tensor ----------------------------------------------------------- */
/*
 * Fake-quantise x [batch, rows, cols] along cols (the weight parametrisation
 * and activation pre-hook of the nxmr.cn article, section 二.3, applied to a
 * whole 3D stack at once, section 二.4), and optionally run the
 * straight-through backward.
 *
 *   q            host; the quantiser.  FQ_NONE copies x.
 *   x            device bf16 [batch, rows, cols]; cols % 8 == 0, 16-B aligned.
 *   scale        device fp32: [batch] (per tensor), [batch, rows] (per row),
 *                [batch, rows, cols/group] (per group; NVFP4: the block scale s_b).
 *                NULL for dynamic sources.
 *   tensor_scale device fp32 [batch]: NVFP4 only (static t for learnable/static
 *                block scales; the learnable t of a dynamic quantiser).
 *   y            device bf16, same shape as x (may alias x); NULL to skip.
 *   codes        device u8, NULL to skip: 4-bit formats [batch, rows, cols/2]
 *                (4-B aligned), 8-bit formats [batch, rows, cols] (8-B aligned).
 *   block_codes  device u8 [batch, rows, cols/16], NVFP4 only; NULL to skip.
 *   grad_y       device dL/dy, bf16 (grad_y_is_fp32 == 0) or fp32, shape of x;
 *                NULL runs the forward only.
 *   grad_x       device bf16 dL/dx (straight-through mask), NULL to skip; needs grad_y.
 *   grad_scale   device fp32 dL/d(parameter), overwritten, NULL to skip; needs
 *                grad_y and a quantiser with a trainable parameter: shape of
 *                `scale` for learnable sources, [batch] for NVFP4 dynamic.
 *   workspace    device scratch of fq_tensor_workspace_size() bytes (may be 0).
 * Errors: FQ_E_INVALID, FQ_E_SHAPE (negative sizes, cols % 8, cols % group),
 * FQ_E_UNSUPPORTED (dynamic per-tensor scales), FQ_E_ALIGN, FQ_E_WORKSPACE, FQ_E_HIP.
 * A zero batch, rows or cols is a no-op.
 */
int fq_tensor(const fq_qdesc* q, int64_t batch, int64_t rows, int64_t cols,
              const void* x, const float* scale, const float* tensor_scale,
              void* y, uint8_t* codes, uint8_t* block_codes,
              const void* grad_y, int32_t grad_y_is_fp32,
              void* grad_x, float* grad_scale,
              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fq_tensor needs for these sizes (0 if none); 0 on bad input. */
size_t fq_tensor_workspace_size(const fq_qdesc* q, int64_t batch, int64_t rows, int64_t cols);

/* ---- the grouped SwiGLU expert layer -------------------------------------- */
/*
 * Per routed copy of token t in slot j, expert e = topk_ids[t, j]:
 *   x^  = fq_a1,e(x[t])                       (activation quantiser of expert e)
 *   z1  = bf16(x^ W1^[e]^T), g = z1[:I], u = z1[I:]
 *   h   = bf16(silu(g) * u), h^ = fq_a2,e(h)
 *   y_r = bf16(h^ W2^[e]^T)
 *   y[t] = bf16(sum_j topk_w[t, j] * y_r)     (fp32, ascending j)
 * with W^ = fq_w(W) over the whole 3D stack.  The router is not quantised:
 * topk_ids / topk_w are inputs (nxmr.cn article, section 二.3).  A quantiser
 * with kind FQ_NONE is the identity, so all-FQ_NONE is the BF16 teacher forward
 * (AngelSlim page, opening paragraph).
 * silu(g) = g / (1 + e^-g) is evaluated in fp32 to within (8 + 2|g|) 2^-24 of
 * its exact value, relative (results below 2^-126 within that plus a subnormal
 * ulp); h therefore equals bf16 of the exact product except where the exact
 * value lies that close to a bf16 rounding midpoint.
 */
typedef struct {
    int64_t E;        /* experts, 1..1024                                        */
    int64_t H;        /* hidden size, multiple of 128                             */
    int64_t I;        /* expert intermediate size, multiple of 128                */
    int64_t T;        /* tokens, >= 0                                             */
    int64_t topk;     /* routed experts per token, 1..min(E, 64)                  */
    fq_qdesc w1, w2;  /* weight quantisers of fc1 (gate|up) and fc2 (down)        */
    fq_qdesc a1, a2;  /* input quantisers of fc1 and fc2 (per expert):
                         FQ_NONE, NVFP4 dynamic, INT/FP8 per-row dynamic, or
                         INT/FP8 per-tensor learnable/static                       */
} fq_layer_desc;

typedef struct {
    const void* w1;     /* device bf16 [E, 2I, H], frozen; rows [0,I) gate, [I,2I) up */
    const void* w2;     /* device bf16 [E, H, I], frozen                               */
    const float* s_w1;  /* device fp32 scale of fc1's weight quantiser (fq_tensor layout, batch = E) */
    const float* t_w1;  /* device fp32 [E] NVFP4 tensor scale of W1, else NULL        */
    const float* s_w2;
    const float* t_w2;
    const float* s_a1;  /* device fp32 [E]: NVFP4 tensor scale or INT/FP8 per-tensor scale; NULL if dynamic per token */
    const float* s_a2;
} fq_expert_params;

typedef struct {        /* device fp32, same shapes as the parameters; NULL to skip */
    float* ds_w1;
    float* ds_w2;
    float* ds_a1;
    float* ds_a2;
} fq_expert_grads;

/* Bytes of the buffer the forward fills for the backward, and of the scratch
 * workspace of each call (0 on an invalid descriptor). */
size_t fq_grouped_expert_saved_size(const fq_layer_desc* L);
size_t fq_grouped_expert_workspace_size(const fq_layer_desc* L);

/*
 * Forward.  x device bf16 [T, H]; topk_ids device int32 [T, topk]; topk_w
 * device fp32 [T, topk]; y device bf16 [T, H] (these may be NULL when T == 0).  `saved` (>= saved_size bytes,
 * 256-B aligned) receives the routing, W^, x^, z1, h^ and y_r for the backward.
 * Errors: FQ_E_INVALID, FQ_E_SHAPE, FQ_E_UNSUPPORTED, FQ_E_ALIGN,
 * FQ_E_WORKSPACE, FQ_E_HIP.
 */
int fq_grouped_expert_fwd(const fq_layer_desc* L, const fq_expert_params* P,
                          const void* x, const int32_t* topk_ids, const float* topk_w,
                          void* y, void* saved, size_t saved_bytes,
                          void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events);

/*
 * `events` (forward and backward): NULL, or a host array of hipEvent_t handles
 * (created by the caller) recorded on `stream` at stage boundaries, for timing:
 * events[i] before stage i and events[n] after the last.  NULL entries are
 * skipped; a skipped stage still records its boundary.
 *   forward  (n = FQ_FWD_STAGES): route, W1 fake-quant, W2 fake-quant,
 *            permute + A1, fc1 GEMM, SwiGLU + A2, fc2 GEMM, combine
 *   backward (n = FQ_BWD_STAGES): permute dY, fc2 dgrad, fc2 wgrad, SwiGLU + A2
 *            backward, A2 scale sum, fc1 dgrad, fc1 wgrad, A1 backward +
 *            unpermute, A1 scale sum, W1 scale grad, W2 scale grad
 */
enum { FQ_FWD_STAGES = 8, FQ_BWD_STAGES = 11 };

/*
 * Straight-through backward from dy (device bf16 [T, H]) and the forward's
 * `saved` buffer (same x, ids, weights and parameters as the forward).
 *   dx        device bf16 [T, H] dL/dx, NULL to skip.
 *   d_topk_w  device fp32 [T, topk] dL/dtopk_w, NULL to skip.
 *   G         host struct of device gradient pointers; each NULL to skip; a
 *             non-NULL pointer for a quantiser without a trainable parameter
 *             is FQ_E_INVALID.
 * The frozen weights get no gradient (AngelSlim page, opening paragraph).
 */
int fq_grouped_expert_bwd(const fq_layer_desc* L, const fq_expert_params* P,
                          const void* x, const int32_t* topk_ids, const float* topk_w,
                          const void* dy, const void* saved, size_t saved_bytes,
                          void* dx, float* d_topk_w, const fq_expert_grads* G,
                          void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events);

/* Location of an intermediate inside `saved` (FQ_BUF_* < 100) or the backward's
 * workspace (>= 100), for inspection between calls: *offset and *bytes.
 * Errors: FQ_E_INVALID for an unknown id or an invalid descriptor. */
typedef enum {
    FQ_BUF_COUNTS = 0,   /* int32 [E] rows per expert                         */
    FQ_BUF_OFFSETS = 1,  /* int32 [E+1] exclusive prefix sum of counts        */
    FQ_BUF_ROW_OF = 2,   /* int32 [T*topk] routed row of flat index t*topk+j  */
    FQ_BUF_SRC_OF = 3,   /* int32 [T*topk] flat index held by routed row r    */
    FQ_BUF_W1HAT = 4,    /* bf16 [E, 2I, H]                                    */
    FQ_BUF_W2HAT = 5,    /* bf16 [E, H, I]                                     */
    FQ_BUF_XHAT = 6,     /* bf16 [T*topk, H] routed rows, experts ascending    */
    FQ_BUF_Z1 = 7,       /* bf16 [T*topk, 2I]                                  */
    FQ_BUF_HHAT = 8,     /* bf16 [T*topk, I]                                   */
    FQ_BUF_YR = 9,       /* bf16 [T*topk, H]                                   */
    FQ_BUF_DYR = 100,    /* bf16 [T*topk, H]  w * dY, permuted                 */
    FQ_BUF_DHHAT = 101,  /* bf16 [T*topk, I]                                   */
    FQ_BUF_DZ1 = 102,    /* bf16 [T*topk, 2I]                                  */
    FQ_BUF_DXHAT = 103,  /* bf16 [T*topk, H]                                   */
    FQ_BUF_DW1HAT = 104, /* fp32 [E, 2I, H]; 0 bytes where ds_w1 is formed in the GEMM */
    FQ_BUF_DW2HAT = 105  /* fp32 [E, H, I];  0 bytes where ds_w2 is formed in the GEMM */
} fq_buffer;
/* The weight gradient dW^ is an intermediate of the weight-scale gradient only
 * (the weights are frozen).  For learnable NVFP4 weights and for learnable or
 * static INT/FP8 weights with per-tensor, per-row or per-group (16 or >= 32)
 * scales, the scale gradient is reduced in the weight-gradient GEMM's epilogue
 * and dW^ never reaches memory; otherwise (dynamic sources, group 8) it is
 * stored and reduced by the fake-quant backward. */
int fq_grouped_expert_buffer(const fq_layer_desc* L, int32_t which, size_t* offset, size_t* bytes);

/* ---- scale optimiser step --------------------------------------------------
 * One AdamW step over the learnable quantiser scales (the only trained
 * parameters), all gradients first clipped by their global L2 norm.  The
 * settings are those of the AngelSlim "MCoreQAD Backend" page ("Train from
 * YAML", the optim block: lr 2e-4, weight decay 0, betas (0.9, 0.95), grad clip
 * 1.0; the nxmr.cn article, section 四, notes that scale-only training takes
 * this higher rate).  The pages name no algorithm; betas with decoupled decay
 * are read as AdamW in PyTorch's documented form (eps 1e-8):
 *     c = min(1, max_grad_norm / (||g|| + 1e-6))     (c = 1 if max_grad_norm <= 0)
 *     g' = c g;   m = b1 m + (1 - b1) g';   v = b2 v + (1 - b2) g'^2
 *     p = p (1 - lr wd) - (lr / (1 - b1^step)) m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * with ||g|| over every tensor of the call.  The updated scale is then kept
 * usable by the forward: an NVFP4 block scale clamped into
 * [t 2^-9, t 448] of its tensor scale t (s / t then casts to a finite,
 * non-zero E4M3 value), any other scale to >= 2^-126.
 * Arithmetic is fp32 (norm in fp64); the result is bitwise deterministic.
 * Tensors of one call must not overlap, except that tensor_scale may be any
 * read-only array. */
#define FQ_MAX_SCALE_PARAMS 16
typedef enum {
    FQ_PROJ_POSITIVE = 0,   /* p >= 2^-126                                        */
    FQ_PROJ_E4M3_BLOCK = 1  /* NVFP4 block scales: t 2^-9 <= p <= t 448           */
} fq_scale_proj;
typedef struct {
    float* param;              /* device fp32 [count], updated in place            */
    const float* grad;         /* device fp32 [count]                              */
    float* exp_avg;            /* device fp32 [count], m; zero before step 1       */
    float* exp_avg_sq;         /* device fp32 [count], v; zero before step 1       */
    int64_t count;             /* >= 0                                             */
    int32_t proj;              /* fq_scale_proj                                    */
    const float* tensor_scale; /* FQ_PROJ_E4M3_BLOCK: device fp32, element i uses
                                  tensor_scale[i / per_tensor]; else ignored       */
    int64_t per_tensor;        /* FQ_PROJ_E4M3_BLOCK: >= 1                         */
} fq_scale_param;
typedef struct {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
} fq_adamw_hparams;
/* host: the pages' values (lr 2e-4, betas 0.9 / 0.95, weight decay 0, clip 1.0)
 * and eps 1e-8 */
int fq_adamw_defaults(fq_adamw_hparams* h);
/* bytes of device workspace fq_scale_adamw needs (8-byte aligned) */
size_t fq_scale_adamw_workspace_size(const fq_scale_param* params, int32_t nparams);
/* params: host array of nparams (1 .. FQ_MAX_SCALE_PARAMS) descriptors; h: host;
 * step: 1 for the first step (bias corrections); grad_norm: nullable device fp32
 * [1], receives ||g|| before clipping.  Errors: FQ_E_INVALID for null or
 * non-finite arguments, betas outside [0, 1), eps <= 0, negative lr, weight
 * decay or count, step < 1, a bad proj or per_tensor; FQ_E_ALIGN for pointers
 * not 4-byte aligned (workspace: 8); FQ_E_WORKSPACE if workspace_bytes is short. */
int fq_scale_adamw(const fq_scale_param* params, int32_t nparams, const fq_adamw_hparams* h, int64_t step,
                   float* grad_norm, void* workspace, size_t workspace_bytes, void* stream);

/* The same step with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc.  It allocates nothing: its scratch
 * (the norm pass's partials and the clip factor, 8 bytes per 32768 scale
 * elements of each tensor, rounded up per tensor) is a fixed device array of
 * FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS + 1 doubles (256 KB + 8 B) inside the
 * library, which every GPU the library runs on holds until the process ends.
 * Each call on a GPU uses that GPU's one array, so calls that overlap on one
 * GPU (different streams, or threads) race and must be ordered by the
 * caller; results are otherwise identical, bit for bit, to fq_scale_adamw's.
 * Errors: those of fq_scale_adamw (without the workspace ones), and
 * FQ_E_WORKSPACE when the tensors need more than
 * FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS blocks (about 1.07e9 elements in all);
 * FQ_E_HIP if the array's device address cannot be looked up. */
#define FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS 32768
int fq_scale_adamw_noalloc(const fq_scale_param* params, int32_t nparams, const fq_adamw_hparams* h,
                           int64_t step, float* grad_norm, void* stream);

/* ---- distillation losses ---------------------------------------------------
 * The loss of quantisation-aware distillation on one batch of logits, and its
 * gradient on the student's logits (the nxmr.cn article, section 二.5:
 * total = lm_weight * lm_loss + distill_weight * distill_loss, distill_type kl,
 * rkl or cakld, and with distill_topk > 0 the KL only over the teacher's
 * top-k tokens so that the [tokens, vocab] teacher tensor never exists; the
 * AngelSlim page, "Train from YAML").  The teacher is the same frozen model
 * with its quantisers disabled (FQ_NONE descriptors in this library).
 * Readings (the pages give no formulas): temperature 1; every term is the
 * mean over tokens; lm_loss is the cross entropy of the student at the label;
 * with p the teacher's and q the student's softmax:
 *     kl = KL(p || q), rkl = KL(q || p),
 *     cakld = c kl + (1 - c) rkl, c = max_v p (the teacher's confidence);
 *     top-k kl = sum over the k given ids of p~ (log p~ - log q), p~ the softmax
 *     of the teacher's k logits, log q the student's full log-softmax there.
 * Arithmetic fp32, reductions in a fixed order: bitwise deterministic. */
typedef enum {
    FQ_DISTILL_KL = 0,
    FQ_DISTILL_RKL = 1,
    FQ_DISTILL_CAKLD = 2,
    FQ_DISTILL_TOPK_KL = 3
} fq_distill_type;
typedef struct {
    int32_t type;              /* fq_distill_type                                     */
    int32_t topk;              /* FQ_DISTILL_TOPK_KL: k in [1, 64]; else 0            */
    float lm_weight;           /* weight of the LM cross entropy (needs labels)       */
    float distill_weight;      /* weight of the distillation term                     */
} fq_distill_desc;
/* bytes of device workspace: one fp32 per token (row losses) unless the caller
 * passes row_loss */
size_t fq_distill_workspace_size(int64_t tokens);
/* student_logits: device bf16 [tokens, vocab], vocab % 8 == 0, 16-B aligned.
 * teacher_logits: device bf16 [tokens, vocab] for kl / rkl / cakld, else NULL.
 * teacher_topk_logits / teacher_topk_ids: device fp32 / int32 [tokens, topk]
 *   for the top-k kl (ids distinct and in [0, vocab)), else NULL.
 * labels: nullable device int32 [tokens] in [0, vocab): adds the LM term.
 * loss: device fp32 [1], the mean total loss.  row_loss: nullable device fp32
 *   [tokens], each token's total loss.  grad: nullable device bf16
 *   [tokens, vocab], d loss / d student_logits (16-B aligned).
 * With tokens == 0 the logits may be NULL and loss receives 0.
 * Errors: FQ_E_INVALID (nulls, bad type or topk, non-finite weights),
 * FQ_E_SHAPE (tokens < 0, vocab < 8 or not a multiple of 8, vocab >= 2^31),
 * FQ_E_ALIGN, FQ_E_WORKSPACE. */
int fq_distill_loss(const fq_distill_desc* d, int64_t tokens, int64_t vocab, const void* student_logits,
                    const void* teacher_logits, const float* teacher_topk_logits,
                    const int32_t* teacher_topk_ids, const int32_t* labels, float* loss, float* row_loss,
                    void* grad, void* workspace, size_t workspace_bytes, void* stream);

/* ---- diagnostics ----------------------------------------------------------- */
const char* fq_status_string(int32_t status);   /* static string                */
const char* fq_last_hip_error(void);            /* thread-local; after FQ_E_HIP */
int32_t fq_abi_version(void);                   /* 1                            */

#ifdef __cplusplus
}
#endif
#endif /* FQ_H */
