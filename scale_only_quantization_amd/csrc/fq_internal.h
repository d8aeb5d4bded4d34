// Internal launch interface between the C ABI (fq_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

// One quantiser, resolved on the host.
struct QParams {
    int kind, gran, group, source;
    float qmin, qmax;      // grid bounds (NVFP4 +-6, FP8 +-448, INT [qmin, qmax])
    float qdiv;            // dynamic INT/FP8: amax divisor (qmax or 448)
};

// fq_tensor over [batch, rows, cols].
struct TensorArgs {
    QParams q;
    int64_t batch, rows, cols;
    const uint16_t* x;
    const float* scale;
    const float* tscale;
    uint16_t* y;
    uint8_t* codes;
    uint8_t* bcodes;
    const void* gy;
    int gy_fp32;
    uint16_t* gx;
    float* gscale;
    float* rowpart;        // workspace [batch * rows] (per-tensor gradients)
};

hipError_t launch_tensor_fwd(const TensorArgs& a, hipStream_t st);
hipError_t launch_tensor_bwd(const TensorArgs& a, hipStream_t st);
size_t tensor_workspace_bytes(const QParams& q, int64_t batch, int64_t rows);

// ------------------------------------------------------------------ layer ---
// Row-tile tables of the routed rows, one per GEMM tile height (128, 256):
// tile i covers rows [row0[i], row0[i] + height) of expert[i], clipped to it.
struct TileTable {
    int32_t* tile_expert;  // [max_mtiles(R, E, height)]
    int32_t* tile_row0;
    int32_t* num_tiles;    // [1]
};
constexpr int TILE_HEIGHTS[2] = {128, 256};

struct RouteArgs {
    const int32_t* ids;    // [R]
    int64_t R;
    int E;
    int32_t* counts;       // [E]
    int32_t* offsets;      // [E+1]
    int32_t* row_of;       // [R]
    int32_t* src_of;       // [R]
    int32_t* row_expert;   // [R] expert of each routed row
    TileTable tables[2];   // heights 128 and 256
    int32_t* order;        // [E] experts by descending count
    int32_t* wg_list;      // [8, E] experts of each XCD's weight-gradient work, descending
    int32_t* wg_cnt;       // [8] experts per XCD
    int32_t* hist;         // workspace [nblk, E]
    int32_t* local_rank;   // workspace [R]
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
int64_t route_blocks(int64_t R);
int64_t max_mtiles(int64_t R, int E, int height);

// Activation quantiser of the layer (per expert parameter vector or none).
struct ActQ {
    QParams q;
    const float* s;        // [E] per-expert scale (NVFP4 tensor scale / INT-FP8 per-tensor), or null
};

struct PermuteArgs {       // x [T,H] -> xhat rows (fq_a1 per expert)
    const uint16_t* x;
    const int32_t* ids;
    const int32_t* row_of;
    uint16_t* xhat;
    int64_t T;
    int k, H, E;
    ActQ a1;
};
hipError_t launch_permute_a1(const PermuteArgs& a, hipStream_t st);

struct SwigluArgs {        // z1 [R, 2I] -> hhat [R, I] (fq_a2 per expert)
    const uint16_t* z1;
    const int32_t* row_expert;
    uint16_t* hhat;
    int64_t R;
    int I, E;
    ActQ a2;
};
hipError_t launch_swiglu_a2(const SwigluArgs& a, hipStream_t st);

struct CombineArgs {       // y[t] = sum_j w y_r[row_of]
    const uint16_t* yr;
    const int32_t* row_of;
    const float* w;
    uint16_t* y;
    int64_t T;
    int k, H;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

struct PermuteDyArgs {     // dY_r[row] = w dY[t]; dw = <dY[t], Y_r[row]>
    const uint16_t* dy;
    const float* w;
    const int32_t* row_of;
    const uint16_t* yr;
    uint16_t* dyr;
    float* dw;
    int64_t T;
    int k, H;
};
hipError_t launch_permute_dy(const PermuteDyArgs& a, hipStream_t st);

struct SwigluBwdArgs {     // (z1, dhhat) -> dz1, per-row partial of ds_a2
    const uint16_t* z1;
    const uint16_t* dhh;
    const int32_t* row_expert;
    uint16_t* dz1;
    float* rowpart;        // [R] or null
    int64_t R;
    int I, E;
    ActQ a2;
};
hipError_t launch_swiglu_bwd(const SwigluBwdArgs& a, hipStream_t st);

struct UnpermuteArgs {     // dX[t] = sum_j mask * dXhat[row]; per-row partial of ds_a1
    const uint16_t* x;
    const uint16_t* dxh;
    const int32_t* ids;
    const int32_t* row_of;
    uint16_t* dx;          // or null
    float* rowpart;        // [R] or null
    int64_t T;
    int k, H, E;
    ActQ a1;
};
hipError_t launch_unpermute_a1(const UnpermuteArgs& a, hipStream_t st);
// partials of ds_a1 the unpermute writes per routed row (its waves per token)
int unpermute_split(int H);

// ds[e] = sum of the `per` partials of each row in [offsets[e], offsets[e+1]),
// in a fixed order
hipError_t launch_segment_sum(const float* rowpart, const int32_t* offsets, int E, int per,
                              float* out, hipStream_t st);

// ------------------------------------------------------------------ GEMMs ---
// Weight-scale gradient formed in the weight-gradient GEMM's epilogue: for each
// element of dW_e (never stored) recompute c from the frozen weight and its
// scale and reduce g c over the scale's elements.
struct SgArgs {
    QParams q;
    const uint16_t* W;     // [E, N, K] frozen weights of the stack
    const float* scale;    // its scale parameter (NVFP4 block / group / row / tensor)
    const float* tscale;   // NVFP4 tensor scale [E]
    float* out;            // null: store dW instead; else per-16 block gradients
                           // (part32 == 0) or per-32-column partials [E, N, K/32]
    int part32;
};
// How the weight-scale gradient of a quantiser is formed: 0 from a stored dW by
// the fake-quant backward, 1 directly per 16-column block in the epilogue,
// 2 from per-32-column partials of the epilogue.
int sg_mode(const QParams& q);
hipError_t launch_sg_reduce(const QParams& q, const float* part, int64_t E, int64_t N, int64_t K,
                            float* rowpart, float* out, hipStream_t st);

// C = A B^T per expert over the routed rows (forward), A K-contiguous, B [N, K].
struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t lda, ldb, ldc;
    int64_t strideB, strideC;     // per-expert strides (elements)
    int N, K;
    int64_t R;
    int E;
    const int32_t* offsets;
    TileTable tables[2];          // row tiles of height 128 and 256
    const int32_t* tile_expert;   // the table the launched kernel uses
    const int32_t* tile_row0;
    const int32_t* num_tiles;
    const int32_t* order;
    SgArgs sg;                    // WGRAD only
    const int32_t* wg_list;       // WGRAD: [8, E] experts per XCD (routing scan)
    const int32_t* wg_cnt;        // [8]
    int32_t* wg_ctr;              // [8] tile counters, zero at launch
};
hipError_t launch_gemm_fwd(const GemmArgs& g, hipStream_t st);    // B K-contiguous
hipError_t launch_gemm_dgrad(const GemmArgs& g, hipStream_t st);  // B N-contiguous ([K, N])
hipError_t launch_gemm_wgrad(const GemmArgs& g, hipStream_t st);  // C[e] fp32 [N, K] = A_e^T B_e
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t st);

// ------------------------------------------------------- scale optimiser ---
// One AdamW step over up to MAX_SCALE_PARAMS fp32 tensors, gradients clipped by
// their global L2 norm.  The host folds the bias corrections into step_size
// and bc2_sqrt.
constexpr int MAX_SCALE_PARAMS = 16;
constexpr int64_t ADAM_CHUNK = 32768;   // elements per block of the norm pass
struct AdamParam {
    float* p;
    const float* g;
    float* m;
    float* v;
    int64_t n;                    // elements
    int64_t blk0;                 // this tensor's first block of the norm pass
    int32_t proj;                 // 0: >= 2^-126; 1: [t 2^-9, t 448], t = t[i / per_t]
    int32_t vec;                  // 1: 4 elements per access (16-B aligned, n and per_t % 4 == 0)
    const float* t;
    int64_t per_t;
};
struct AdamArgs {
    AdamParam prm[MAX_SCALE_PARAMS];
    int32_t np;
    int64_t nb;                   // blocks of the norm pass, over every tensor
    float b1, b2, one_m_b1, one_m_b2, eps;
    float decay;                  // 1 - lr wd
    float step_size;              // lr / (1 - b1^t)
    float bc2_sqrt;               // sqrt(1 - b2^t)
    double max_norm;              // <= 0: no clipping
    double* part;                 // workspace [nb]: partial sums of g^2
    float* clip;                  // workspace [1]: the factor applied to every gradient
    float* norm_out;              // nullable [1]: the global norm before clipping
};
int64_t adam_norm_blocks(int64_t count);   // norm-pass blocks of one tensor
hipError_t launch_scale_adamw(const AdamArgs& a, hipStream_t st);

// ------------------------------------------------- distillation losses ---
enum DistillKind : int { DK_KL = 0, DK_RKL = 1, DK_CAKLD = 2, DK_TOPK = 3 };
struct DistillArgs {
    int kind;
    int64_t T, V;                 // rows (tokens), vocabulary (multiple of 8)
    const uint16_t* zs;           // bf16 [T, V] student logits
    const uint16_t* zt;           // bf16 [T, V] teacher logits (kl, rkl, cakld)
    const float* top_v;           // fp32 [T, k] the teacher's top-k logits (top-k kl)
    const int32_t* top_i;         // [T, k] their token ids
    int k;
    const int32_t* labels;        // nullable [T]: the LM term
    float lm_w, dist_w, inv_T;
    float* row_loss;              // [T]
    uint16_t* grad;               // nullable bf16 [T, V]
};
// the row losses, their mean into mean_out[0] and, with a.grad, d mean / d zs
hipError_t launch_distill(const DistillArgs& a, float* mean_out, hipStream_t st);

}  // namespace fq
