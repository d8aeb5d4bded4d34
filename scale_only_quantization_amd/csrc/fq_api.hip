// C ABI of the grouped-expert fake-quant library (declarations and the
// documented contract are in include/fq.h).
//
// Host side only: argument validation (always before any HIP call, so every
// error path is testable without a GPU), the layout of the saved and
// workspace buffers, and the launch order of the forward and backward stages.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "fq.h"
#include "fq_internal.h"

using namespace fq;

namespace {

thread_local char g_hip_error[256] = "";

int hip_fail(hipError_t e) {
    const char* s = hipGetErrorString(e);
    int i = 0;
    for (; s && s[i] && i < 255; ++i) g_hip_error[i] = s[i];
    g_hip_error[i] = 0;
    return FQ_E_HIP;
}

#define FQ_TRY(expr)                                       \
    do {                                                   \
        hipError_t _e = (expr);                            \
        if (_e != hipSuccess) return hip_fail(_e);         \
    } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Resolve and check a quantiser descriptor.  Returns FQ_OK or an error.
int check_qdesc(const fq_qdesc* d, QParams* out) {
    if (!d) return FQ_E_INVALID;
    QParams q{};
    q.kind = d->kind;
    q.gran = d->gran;
    q.group = d->group;
    q.source = d->source;
    if (q.kind < FQ_NONE || q.kind > FQ_FP8E4M3) return FQ_E_INVALID;
    if (q.kind == FQ_NONE) {
        *out = q;
        return FQ_OK;
    }
    if (q.gran < FQ_PER_TENSOR || q.gran > FQ_PER_GROUP) return FQ_E_INVALID;
    if (q.source < FQ_LEARNABLE || q.source > FQ_DYNAMIC) return FQ_E_INVALID;
    if (q.kind == FQ_NVFP4) {
        if (q.gran != FQ_PER_GROUP || q.group != 16) return FQ_E_INVALID;
        q.qmin = -6.0f;
        q.qmax = 6.0f;
    } else if (q.kind == FQ_FP8E4M3) {
        q.qmin = -448.0f;
        q.qmax = 448.0f;
        q.qdiv = 448.0f;
    } else {
        if (d->qmin >= 0 || d->qmax <= 0 || d->qmin < -128 || d->qmax > 127) return FQ_E_INVALID;
        q.qmin = (float)d->qmin;
        q.qmax = (float)d->qmax;
        q.qdiv = (float)d->qmax;
    }
    if (q.gran == FQ_PER_GROUP) {
        if (!pow2(q.group) || q.group < 8 || q.group > 512) return FQ_E_INVALID;
    }
    if (q.gran == FQ_PER_TENSOR && q.source == FQ_DYNAMIC) return FQ_E_UNSUPPORTED;
    *out = q;
    return FQ_OK;
}

// Does the quantiser own a trainable tensor (one that can receive a gradient)?
bool has_param(const QParams& q) {
    if (q.kind == FQ_NVFP4) return q.source != FQ_STATIC;
    return q.kind != FQ_NONE && q.source == FQ_LEARNABLE;
}
// Does it read `scale` (the per-tensor/row/group or NVFP4 block scale)?
bool needs_scale(const QParams& q) { return q.kind != FQ_NONE && q.source != FQ_DYNAMIC; }
bool four_bit(const QParams& q) {
    return q.kind == FQ_NVFP4 || (q.kind == FQ_INT && q.qmax - q.qmin < 16.0f);
}

// ------------------------------------------------------------ layer layout --
struct Section {
    size_t off = 0, bytes = 0;
};

struct Layout {
    // saved
    Section counts, offsets, row_of, src_of, row_expert, tile_expert[2], tile_row0[2], num_tiles, order, wg_list, wg_cnt;
    Section w1hat, w2hat, xhat, z1, hhat, yr;
    size_t saved = 0;
    // workspace
    Section hist, local_rank, dyr, dhh, dz1, dxh, dw1, dw2, sgp1, sgp2, rowpart1, rowpart2, tws, wg_ctr;
    size_t ws = 0;
};

void place(Section& s, size_t bytes, size_t& cur) {
    s.off = cur;
    s.bytes = bytes;
    cur = round_up(cur + bytes, 256);
}

struct LayerQ {
    QParams w1, w2, a1, a2;
};

int check_act(const QParams& a, int64_t width) {
    if (a.kind == FQ_NONE) return FQ_OK;
    if (a.kind == FQ_NVFP4) return a.source == FQ_DYNAMIC ? FQ_OK : FQ_E_UNSUPPORTED;
    if (a.source == FQ_DYNAMIC) {
        if (a.gran == FQ_PER_GROUP && width % a.group != 0) return FQ_E_SHAPE;
        return FQ_OK;                                  // per row / per group, on the fly
    }
    return a.gran == FQ_PER_TENSOR ? FQ_OK : FQ_E_UNSUPPORTED;   // per-expert scale
}

int check_layer(const fq_layer_desc* L, LayerQ* q) {
    if (!L) return FQ_E_INVALID;
    if (L->E < 1 || L->E > 1024 || L->H <= 0 || L->I <= 0 || L->T < 0) return FQ_E_SHAPE;
    if (L->topk < 1 || L->topk > 64 || L->topk > L->E) return FQ_E_SHAPE;
    if (L->H % 128 || L->I % 128) return FQ_E_SHAPE;
    if (L->H > 8192 || L->I > 8192) return FQ_E_UNSUPPORTED;
    if (L->T * L->topk >= (int64_t)1 << 31) return FQ_E_SHAPE;
    int s;
    if ((s = check_qdesc(&L->w1, &q->w1)) != FQ_OK) return s;
    if ((s = check_qdesc(&L->w2, &q->w2)) != FQ_OK) return s;
    if ((s = check_qdesc(&L->a1, &q->a1)) != FQ_OK) return s;
    if ((s = check_qdesc(&L->a2, &q->a2)) != FQ_OK) return s;
    if (q->w1.gran == FQ_PER_GROUP && L->H % q->w1.group) return FQ_E_SHAPE;
    if (q->w2.gran == FQ_PER_GROUP && L->I % q->w2.group) return FQ_E_SHAPE;
    if ((s = check_act(q->a1, L->H)) != FQ_OK) return s;
    if ((s = check_act(q->a2, L->I)) != FQ_OK) return s;
    return FQ_OK;
}

Layout layout(const fq_layer_desc* L, const LayerQ& q) {
    Layout y;
    const int64_t E = L->E, H = L->H, I = L->I, R = L->T * L->topk;
    size_t c = 0;
    place(y.counts, E * 4, c);
    place(y.offsets, (E + 1) * 4, c);
    place(y.row_of, R * 4, c);
    place(y.src_of, R * 4, c);
    place(y.row_expert, R * 4, c);
    for (int h = 0; h < 2; ++h) {
        const int64_t mt = max_mtiles(R, (int)E, TILE_HEIGHTS[h]);
        place(y.tile_expert[h], mt * 4, c);
        place(y.tile_row0[h], mt * 4, c);
    }
    place(y.num_tiles, 2 * 4, c);
    place(y.order, E * 4, c);
    place(y.wg_list, 8 * E * 4, c);
    place(y.wg_cnt, 8 * 4, c);
    place(y.w1hat, q.w1.kind != FQ_NONE ? (size_t)E * 2 * I * H * 2 : 0, c);
    place(y.w2hat, q.w2.kind != FQ_NONE ? (size_t)E * H * I * 2 : 0, c);
    place(y.xhat, (size_t)R * H * 2, c);
    place(y.z1, (size_t)R * 2 * I * 2, c);
    place(y.hhat, (size_t)R * I * 2, c);
    place(y.yr, (size_t)R * H * 2, c);
    y.saved = c;
    c = 0;
    place(y.hist, (size_t)route_blocks(R) * E * 4, c);
    place(y.local_rank, R * 4, c);
    place(y.dyr, (size_t)R * H * 2, c);
    place(y.dhh, (size_t)R * I * 2, c);
    place(y.dz1, (size_t)R * 2 * I * 2, c);
    place(y.dxh, (size_t)R * H * 2, c);
    // dW^ is stored only where the weight-scale gradient is not formed in the
    // weight-gradient GEMM's epilogue; per-32-column partials where it is
    const int m1 = sg_mode(q.w1), m2 = sg_mode(q.w2);
    place(y.dw1, q.w1.kind != FQ_NONE && m1 == 0 ? (size_t)E * 2 * I * H * 4 : 0, c);
    place(y.dw2, q.w2.kind != FQ_NONE && m2 == 0 ? (size_t)E * H * I * 4 : 0, c);
    place(y.sgp1, m1 == 2 ? (size_t)E * 2 * I * (H / 32) * 4 : 0, c);
    place(y.sgp2, m2 == 2 ? (size_t)E * H * (I / 32) * 4 : 0, c);
    place(y.rowpart1, R * 4 * unpermute_split((int)L->H), c);
    place(y.rowpart2, R * 4, c);
    const size_t t1 = tensor_workspace_bytes(q.w1, E, 2 * I);
    const size_t t2 = tensor_workspace_bytes(q.w2, E, H);
    place(y.tws, t1 > t2 ? t1 : t2, c);
    place(y.wg_ctr, 16 * 4, c);
    y.ws = c;
    return y;
}

// Check the pointers a quantiser needs in a layer.
int check_wparams(const QParams& q, const void* w, const float* s, const float* t) {
    if (!w) return FQ_E_INVALID;
    if (!aligned(w, 16)) return FQ_E_ALIGN;
    if (needs_scale(q) && !s) return FQ_E_INVALID;
    if (q.kind == FQ_NVFP4 && !t) return FQ_E_INVALID;
    if ((s && !aligned(s, 4)) || (t && !aligned(t, 4))) return FQ_E_ALIGN;
    return FQ_OK;
}
int check_aparams(const QParams& q, const float* s) {
    const bool need = q.kind == FQ_NVFP4 || (q.kind != FQ_NONE && q.source != FQ_DYNAMIC);
    if (need && !s) return FQ_E_INVALID;
    if (s && !aligned(s, 4)) return FQ_E_ALIGN;
    return FQ_OK;
}

// record the caller's stage-boundary event i (if any) on the stream
hipError_t mark(void* const* events, int i, hipStream_t st) {
    if (!events || !events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
}

template <typename T>
T* at(void* base, const Section& s) { return reinterpret_cast<T*>(static_cast<char*>(base) + s.off); }
template <typename T>
const T* at(const void* base, const Section& s) {
    return reinterpret_cast<const T*>(static_cast<const char*>(base) + s.off);
}

}  // namespace

extern "C" {

int32_t fq_abi_version(void) { return 1; }

const char* fq_status_string(int32_t status) {
    switch (status) {
    case FQ_OK: return "ok";
    case FQ_E_INVALID: return "invalid argument";
    case FQ_E_SHAPE: return "invalid shape";
    case FQ_E_UNSUPPORTED: return "unsupported quantiser or shape";
    case FQ_E_WORKSPACE: return "buffer too small";
    case FQ_E_ALIGN: return "misaligned pointer";
    case FQ_E_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char* fq_last_hip_error(void) { return g_hip_error; }

int fq_preset(int32_t format, fq_qdesc* w1, fq_qdesc* w2, fq_qdesc* a1, fq_qdesc* a2) {
    if (!w1 || !w2 || !a1 || !a2) return FQ_E_INVALID;
    const fq_qdesc none = {FQ_NONE, FQ_PER_TENSOR, 0, FQ_LEARNABLE, 0, 0};
    const fq_qdesc nvfp4_w = {FQ_NVFP4, FQ_PER_GROUP, 16, FQ_LEARNABLE, 0, 0};
    const fq_qdesc nvfp4_a = {FQ_NVFP4, FQ_PER_GROUP, 16, FQ_DYNAMIC, 0, 0};
    const fq_qdesc int4_g = {FQ_INT, FQ_PER_GROUP, 128, FQ_LEARNABLE, -8, 7};
    const fq_qdesc int8_row = {FQ_INT, FQ_PER_ROW, 0, FQ_LEARNABLE, -128, 127};
    const fq_qdesc int8_tok = {FQ_INT, FQ_PER_ROW, 0, FQ_DYNAMIC, -128, 127};
    const fq_qdesc fp8_row = {FQ_FP8E4M3, FQ_PER_ROW, 0, FQ_LEARNABLE, 0, 0};
    const fq_qdesc fp8_tok = {FQ_FP8E4M3, FQ_PER_ROW, 0, FQ_DYNAMIC, 0, 0};
    const fq_qdesc fp8_ten = {FQ_FP8E4M3, FQ_PER_TENSOR, 0, FQ_LEARNABLE, 0, 0};
    fq_qdesc w, a;
    switch (format) {
    case FQ_FMT_NVFP4: w = nvfp4_w; a = nvfp4_a; break;
    case FQ_FMT_NVFP4A16: w = nvfp4_w; a = none; break;
    case FQ_FMT_W4A16: w = int4_g; a = none; break;
    case FQ_FMT_W8A8: w = int8_row; a = int8_tok; break;
    case FQ_FMT_FP8: w = fp8_row; a = fp8_tok; break;
    case FQ_FMT_W4AFP8: w = int4_g; a = fp8_ten; break;
    default: return FQ_E_INVALID;
    }
    *w1 = w;
    *w2 = w;
    *a1 = a;
    *a2 = a;
    return FQ_OK;
}

size_t fq_tensor_workspace_size(const fq_qdesc* d, int64_t batch, int64_t rows, int64_t cols) {
    QParams q;
    if (check_qdesc(d, &q) != FQ_OK || batch < 0 || rows < 0 || cols < 0) return 0;
    return tensor_workspace_bytes(q, batch, rows);
}

int fq_tensor(const fq_qdesc* d, int64_t batch, int64_t rows, int64_t cols, const void* x,
              const float* scale, const float* tensor_scale, void* y, uint8_t* codes,
              uint8_t* block_codes, const void* grad_y, int32_t grad_y_is_fp32, void* grad_x,
              float* grad_scale, void* workspace, size_t workspace_bytes, void* stream) {
    QParams q;
    int s = check_qdesc(d, &q);
    if (s != FQ_OK) return s;
    if (batch < 0 || rows < 0 || cols < 0) return FQ_E_SHAPE;
    if (cols % 8) return FQ_E_SHAPE;
    if (q.gran == FQ_PER_GROUP && q.kind != FQ_NONE && cols % q.group) return FQ_E_SHAPE;
    if (batch * rows * cols >= ((int64_t)1 << 40)) return FQ_E_SHAPE;
    if (!x) return FQ_E_INVALID;
    if ((grad_x || grad_scale) && !grad_y) return FQ_E_INVALID;
    if (grad_scale && !has_param(q)) return FQ_E_INVALID;
    if (needs_scale(q) && !scale) return FQ_E_INVALID;
    if (q.kind == FQ_NVFP4 && !tensor_scale) return FQ_E_INVALID;
    if (block_codes && q.kind != FQ_NVFP4) return FQ_E_INVALID;
    if (codes && q.kind == FQ_NONE) return FQ_E_INVALID;
    if (!aligned(x, 16) || (y && !aligned(y, 16)) || (grad_x && !aligned(grad_x, 16)) ||
        (grad_y && !aligned(grad_y, 16)))
        return FQ_E_ALIGN;
    if ((scale && !aligned(scale, 4)) || (tensor_scale && !aligned(tensor_scale, 4)) ||
        (grad_scale && !aligned(grad_scale, 4)))
        return FQ_E_ALIGN;
    if (codes && !aligned(codes, four_bit(q) ? 4 : 8)) return FQ_E_ALIGN;
    const size_t need = grad_scale ? tensor_workspace_bytes(q, batch, rows) : 0;
    if (workspace_bytes < need || (need && !workspace)) return FQ_E_WORKSPACE;
    if (batch == 0 || rows == 0 || cols == 0) return FQ_OK;

    TensorArgs a{};
    a.q = q;
    a.batch = batch;
    a.rows = rows;
    a.cols = cols;
    a.x = static_cast<const uint16_t*>(x);
    a.scale = scale;
    a.tscale = tensor_scale;
    a.y = static_cast<uint16_t*>(y);
    a.codes = codes;
    a.bcodes = block_codes;
    a.gy = grad_y;
    a.gy_fp32 = grad_y_is_fp32 ? 1 : 0;
    a.gx = static_cast<uint16_t*>(grad_x);
    a.gscale = grad_scale;
    a.rowpart = static_cast<float*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (y || codes || block_codes) FQ_TRY(launch_tensor_fwd(a, st));
    if (grad_x || grad_scale) FQ_TRY(launch_tensor_bwd(a, st));
    return FQ_OK;
}

size_t fq_grouped_expert_saved_size(const fq_layer_desc* L) {
    LayerQ q;
    if (check_layer(L, &q) != FQ_OK) return 0;
    return layout(L, q).saved;
}

size_t fq_grouped_expert_workspace_size(const fq_layer_desc* L) {
    LayerQ q;
    if (check_layer(L, &q) != FQ_OK) return 0;
    return layout(L, q).ws;
}

int fq_grouped_expert_buffer(const fq_layer_desc* L, int32_t which, size_t* offset, size_t* bytes) {
    LayerQ q;
    int s = check_layer(L, &q);
    if (s != FQ_OK) return s;
    if (!offset || !bytes) return FQ_E_INVALID;
    const Layout y = layout(L, q);
    const Section* sec = nullptr;
    switch (which) {
    case FQ_BUF_COUNTS: sec = &y.counts; break;
    case FQ_BUF_OFFSETS: sec = &y.offsets; break;
    case FQ_BUF_ROW_OF: sec = &y.row_of; break;
    case FQ_BUF_SRC_OF: sec = &y.src_of; break;
    case FQ_BUF_W1HAT: sec = &y.w1hat; break;
    case FQ_BUF_W2HAT: sec = &y.w2hat; break;
    case FQ_BUF_XHAT: sec = &y.xhat; break;
    case FQ_BUF_Z1: sec = &y.z1; break;
    case FQ_BUF_HHAT: sec = &y.hhat; break;
    case FQ_BUF_YR: sec = &y.yr; break;
    case FQ_BUF_DYR: sec = &y.dyr; break;
    case FQ_BUF_DHHAT: sec = &y.dhh; break;
    case FQ_BUF_DZ1: sec = &y.dz1; break;
    case FQ_BUF_DXHAT: sec = &y.dxh; break;
    case FQ_BUF_DW1HAT: sec = &y.dw1; break;
    case FQ_BUF_DW2HAT: sec = &y.dw2; break;
    default: return FQ_E_INVALID;
    }
    *offset = sec->off;
    *bytes = sec->bytes;
    return FQ_OK;
}

int fq_grouped_expert_fwd(const fq_layer_desc* L, const fq_expert_params* P, const void* x,
                          const int32_t* topk_ids, const float* topk_w, void* y, void* saved,
                          size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events) {
    LayerQ q;
    int s = check_layer(L, &q);
    if (s != FQ_OK) return s;
    if (!P || !saved) return FQ_E_INVALID;
    if (L->T > 0 && (!x || !topk_ids || !topk_w || !y)) return FQ_E_INVALID;   // may be NULL when empty
    if ((s = check_wparams(q.w1, P->w1, P->s_w1, P->t_w1)) != FQ_OK) return s;
    if ((s = check_wparams(q.w2, P->w2, P->s_w2, P->t_w2)) != FQ_OK) return s;
    if ((s = check_aparams(q.a1, P->s_a1)) != FQ_OK) return s;
    if ((s = check_aparams(q.a2, P->s_a2)) != FQ_OK) return s;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
        !aligned(saved, 256) || (workspace && !aligned(workspace, 256)))
        return FQ_E_ALIGN;
    const Layout lay = layout(L, q);
    if (saved_bytes < lay.saved) return FQ_E_WORKSPACE;
    if (workspace_bytes < lay.ws || (lay.ws && !workspace)) return FQ_E_WORKSPACE;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int E = (int)L->E, H = (int)L->H, I = (int)L->I, k = (int)L->topk;
    const int64_t T = L->T, R = T * k;

    RouteArgs ra{};
    ra.ids = topk_ids;
    ra.R = R;
    ra.E = E;
    ra.counts = at<int32_t>(saved, lay.counts);
    ra.offsets = at<int32_t>(saved, lay.offsets);
    ra.row_of = at<int32_t>(saved, lay.row_of);
    ra.src_of = at<int32_t>(saved, lay.src_of);
    ra.row_expert = at<int32_t>(saved, lay.row_expert);
    for (int h = 0; h < 2; ++h) {
        ra.tables[h].tile_expert = at<int32_t>(saved, lay.tile_expert[h]);
        ra.tables[h].tile_row0 = at<int32_t>(saved, lay.tile_row0[h]);
        ra.tables[h].num_tiles = at<int32_t>(saved, lay.num_tiles) + h;
    }
    ra.order = at<int32_t>(saved, lay.order);
    ra.wg_list = at<int32_t>(saved, lay.wg_list);
    ra.wg_cnt = at<int32_t>(saved, lay.wg_cnt);
    ra.hist = at<int32_t>(workspace, lay.hist);
    ra.local_rank = at<int32_t>(workspace, lay.local_rank);
    FQ_TRY(mark(events, 0, st));
    FQ_TRY(launch_route(ra, st));

    // F3: the whole weight stacks in one pass each
    FQ_TRY(mark(events, 1, st));
    const uint16_t* w1h = static_cast<const uint16_t*>(P->w1);
    const uint16_t* w2h = static_cast<const uint16_t*>(P->w2);
    if (q.w1.kind != FQ_NONE) {
        TensorArgs ta{};
        ta.q = q.w1;
        ta.batch = E;
        ta.rows = 2 * I;
        ta.cols = H;
        ta.x = w1h;
        ta.scale = P->s_w1;
        ta.tscale = P->t_w1;
        ta.y = at<uint16_t>(saved, lay.w1hat);
        FQ_TRY(launch_tensor_fwd(ta, st));
        w1h = ta.y;
    }
    FQ_TRY(mark(events, 2, st));
    if (q.w2.kind != FQ_NONE) {
        TensorArgs ta{};
        ta.q = q.w2;
        ta.batch = E;
        ta.rows = H;
        ta.cols = I;
        ta.x = w2h;
        ta.scale = P->s_w2;
        ta.tscale = P->t_w2;
        ta.y = at<uint16_t>(saved, lay.w2hat);
        FQ_TRY(launch_tensor_fwd(ta, st));
        w2h = ta.y;
    }

    // F2: permute + A1
    PermuteArgs pa{};
    pa.x = static_cast<const uint16_t*>(x);
    pa.ids = topk_ids;
    pa.row_of = ra.row_of;
    pa.xhat = at<uint16_t>(saved, lay.xhat);
    pa.T = T;
    pa.k = k;
    pa.H = H;
    pa.E = E;
    pa.a1 = ActQ{q.a1, P->s_a1};
    FQ_TRY(mark(events, 3, st));
    FQ_TRY(launch_permute_a1(pa, st));

    // F4: fc1
    GemmArgs g{};
    g.R = R;
    g.E = E;
    g.offsets = ra.offsets;
    g.tables[0] = ra.tables[0];
    g.tables[1] = ra.tables[1];
    g.order = ra.order;
    g.A = pa.xhat;
    g.lda = H;
    g.B = w1h;
    g.ldb = H;
    g.strideB = (int64_t)2 * I * H;
    g.C = at<uint16_t>(saved, lay.z1);
    g.ldc = 2 * I;
    g.N = 2 * I;
    g.K = H;
    FQ_TRY(mark(events, 4, st));
    FQ_TRY(launch_gemm_fwd(g, st));

    // F5: SwiGLU + A2
    SwigluArgs sa{};
    sa.z1 = at<uint16_t>(saved, lay.z1);
    sa.row_expert = ra.row_expert;
    sa.hhat = at<uint16_t>(saved, lay.hhat);
    sa.R = R;
    sa.I = I;
    sa.E = E;
    sa.a2 = ActQ{q.a2, P->s_a2};
    FQ_TRY(mark(events, 5, st));
    FQ_TRY(launch_swiglu_a2(sa, st));

    // F6: fc2
    g.A = sa.hhat;
    g.lda = I;
    g.B = w2h;
    g.ldb = I;
    g.strideB = (int64_t)H * I;
    g.C = at<uint16_t>(saved, lay.yr);
    g.ldc = H;
    g.N = H;
    g.K = I;
    FQ_TRY(mark(events, 6, st));
    FQ_TRY(launch_gemm_fwd(g, st));

    // F7: combine
    CombineArgs ca{};
    ca.yr = at<uint16_t>(saved, lay.yr);
    ca.row_of = ra.row_of;
    ca.w = topk_w;
    ca.y = static_cast<uint16_t*>(y);
    ca.T = T;
    ca.k = k;
    ca.H = H;
    FQ_TRY(mark(events, 7, st));
    FQ_TRY(launch_combine(ca, st));
    FQ_TRY(mark(events, FQ_FWD_STAGES, st));
    return FQ_OK;
}

int fq_grouped_expert_bwd(const fq_layer_desc* L, const fq_expert_params* P, const void* x,
                          const int32_t* topk_ids, const float* topk_w, const void* dy,
                          const void* saved, size_t saved_bytes, void* dx, float* d_topk_w,
                          const fq_expert_grads* G, void* workspace, size_t workspace_bytes,
                          void* stream, void* const* events) {
    LayerQ q;
    int s = check_layer(L, &q);
    if (s != FQ_OK) return s;
    if (!P || !saved || !G) return FQ_E_INVALID;
    if (L->T > 0 && (!x || !topk_ids || !topk_w || !dy)) return FQ_E_INVALID;  // may be NULL when empty
    if ((s = check_wparams(q.w1, P->w1, P->s_w1, P->t_w1)) != FQ_OK) return s;
    if ((s = check_wparams(q.w2, P->w2, P->s_w2, P->t_w2)) != FQ_OK) return s;
    if ((s = check_aparams(q.a1, P->s_a1)) != FQ_OK) return s;
    if ((s = check_aparams(q.a2, P->s_a2)) != FQ_OK) return s;
    if ((G->ds_w1 && !has_param(q.w1)) || (G->ds_w2 && !has_param(q.w2)) ||
        (G->ds_a1 && !has_param(q.a1)) || (G->ds_a2 && !has_param(q.a2)))
        return FQ_E_INVALID;
    if (!aligned(x, 16) || !aligned(dy, 16) || (dx && !aligned(dx, 16)) || !aligned(topk_ids, 4) ||
        !aligned(topk_w, 4) || (d_topk_w && !aligned(d_topk_w, 4)) || !aligned(saved, 256) ||
        (workspace && !aligned(workspace, 256)))
        return FQ_E_ALIGN;
    if ((G->ds_w1 && !aligned(G->ds_w1, 4)) || (G->ds_w2 && !aligned(G->ds_w2, 4)) ||
        (G->ds_a1 && !aligned(G->ds_a1, 4)) || (G->ds_a2 && !aligned(G->ds_a2, 4)))
        return FQ_E_ALIGN;
    const Layout lay = layout(L, q);
    if (saved_bytes < lay.saved) return FQ_E_WORKSPACE;
    if (workspace_bytes < lay.ws || (lay.ws && !workspace)) return FQ_E_WORKSPACE;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int E = (int)L->E, H = (int)L->H, I = (int)L->I, k = (int)L->topk;
    const int64_t T = L->T, R = T * k;
    const int32_t* offsets = at<int32_t>(saved, lay.offsets);
    const int32_t* row_of = at<int32_t>(saved, lay.row_of);
    const int32_t* src_of = at<int32_t>(saved, lay.src_of);
    const uint16_t* w1h = q.w1.kind != FQ_NONE ? at<uint16_t>(saved, lay.w1hat) : static_cast<const uint16_t*>(P->w1);
    const uint16_t* w2h = q.w2.kind != FQ_NONE ? at<uint16_t>(saved, lay.w2hat) : static_cast<const uint16_t*>(P->w2);
    uint16_t* dyr = at<uint16_t>(workspace, lay.dyr);
    uint16_t* dhh = at<uint16_t>(workspace, lay.dhh);
    uint16_t* dz1 = at<uint16_t>(workspace, lay.dz1);
    uint16_t* dxh = at<uint16_t>(workspace, lay.dxh);
    float* dw1 = at<float>(workspace, lay.dw1);
    float* dw2 = at<float>(workspace, lay.dw2);
    const int m1 = sg_mode(q.w1), m2 = sg_mode(q.w2);
    // the fused weight-scale gradient of one stack: W, its scales, and where
    // the epilogue writes (the gradient itself, or partials)
    auto sg_of = [&](const QParams& qq, int m, const void* W, const float* sc, const float* ts, float* ds,
                     const Section& part) {
        SgArgs a{};
        if (m == 0 || !ds) return a;
        a.q = qq;
        a.W = static_cast<const uint16_t*>(W);
        a.scale = sc;
        a.tscale = ts;
        a.part32 = m == 2;
        a.out = m == 2 ? at<float>(workspace, part) : ds;
        return a;
    };

    // B1: permute dY (and the routing-weight gradient)
    PermuteDyArgs pd{};
    pd.dy = static_cast<const uint16_t*>(dy);
    pd.w = topk_w;
    pd.row_of = row_of;
    pd.yr = at<uint16_t>(saved, lay.yr);
    pd.dyr = dyr;
    pd.dw = d_topk_w;
    pd.T = T;
    pd.k = k;
    pd.H = H;
    FQ_TRY(mark(events, 0, st));
    FQ_TRY(launch_permute_dy(pd, st));

    GemmArgs g{};
    g.R = R;
    g.E = E;
    g.offsets = offsets;
    for (int h = 0; h < 2; ++h) {
        g.tables[h].tile_expert = const_cast<int32_t*>(at<int32_t>(saved, lay.tile_expert[h]));
        g.tables[h].tile_row0 = const_cast<int32_t*>(at<int32_t>(saved, lay.tile_row0[h]));
        g.tables[h].num_tiles = const_cast<int32_t*>(at<int32_t>(saved, lay.num_tiles)) + h;
    }
    g.order = at<int32_t>(saved, lay.order);
    g.wg_list = at<int32_t>(saved, lay.wg_list);
    g.wg_cnt = at<int32_t>(saved, lay.wg_cnt);
    int32_t* wg_ctr = at<int32_t>(workspace, lay.wg_ctr);     // fc2, fc1 weight-gradient tile counters
    if (G->ds_w1 || G->ds_w2) FQ_TRY(launch_zero_i32(wg_ctr, 16, st));

    // B2: fc2 dgrad  dH^ = dY_r W2^
    g.A = dyr;
    g.lda = H;
    g.B = w2h;
    g.ldb = I;
    g.strideB = (int64_t)H * I;
    g.C = dhh;
    g.ldc = I;
    g.N = I;
    g.K = H;
    FQ_TRY(mark(events, 1, st));
    FQ_TRY(launch_gemm_dgrad(g, st));

    FQ_TRY(mark(events, 2, st));
    // B3: fc2 wgrad  dW2^ = dY_r^T H^ (only to form the weight-scale gradient)
    if (G->ds_w2) {
        g.A = dyr;
        g.lda = H;
        g.B = at<uint16_t>(saved, lay.hhat);
        g.ldb = I;
        g.C = dw2;
        g.ldc = I;
        g.strideC = (int64_t)H * I;
        g.N = H;
        g.K = I;
        g.sg = sg_of(q.w2, m2, P->w2, P->s_w2, P->t_w2, G->ds_w2, lay.sgp2);
        g.wg_ctr = wg_ctr;
        FQ_TRY(launch_gemm_wgrad(g, st));
        g.sg = SgArgs{};
    }

    // B4: A2 straight-through + SwiGLU backward
    SwigluBwdArgs sb{};
    sb.z1 = at<uint16_t>(saved, lay.z1);
    sb.dhh = dhh;
    sb.row_expert = at<int32_t>(saved, lay.row_expert);
    sb.dz1 = dz1;
    sb.rowpart = G->ds_a2 ? at<float>(workspace, lay.rowpart2) : nullptr;
    sb.R = R;
    sb.I = I;
    sb.E = E;
    sb.a2 = ActQ{q.a2, P->s_a2};
    FQ_TRY(mark(events, 3, st));
    FQ_TRY(launch_swiglu_bwd(sb, st));
    FQ_TRY(mark(events, 4, st));
    if (G->ds_a2) FQ_TRY(launch_segment_sum(sb.rowpart, offsets, E, 1, G->ds_a2, st));
    FQ_TRY(mark(events, 5, st));

    const bool need_dxh = dx || G->ds_a1;
    if (need_dxh) {
        // B5: fc1 dgrad  dX^ = dZ1 W1^
        g.A = dz1;
        g.lda = 2 * I;
        g.B = w1h;
        g.ldb = H;
        g.strideB = (int64_t)2 * I * H;
        g.C = dxh;
        g.ldc = H;
        g.N = H;
        g.K = 2 * I;
        FQ_TRY(launch_gemm_dgrad(g, st));
    }
    FQ_TRY(mark(events, 6, st));
    if (G->ds_w1) {
        // B6: fc1 wgrad  dW1^ = dZ1^T X^
        g.A = dz1;
        g.lda = 2 * I;
        g.B = at<uint16_t>(saved, lay.xhat);
        g.ldb = H;
        g.C = dw1;
        g.ldc = H;
        g.strideC = (int64_t)2 * I * H;
        g.N = 2 * I;
        g.K = H;
        g.sg = sg_of(q.w1, m1, P->w1, P->s_w1, P->t_w1, G->ds_w1, lay.sgp1);
        g.wg_ctr = wg_ctr + 8;
        FQ_TRY(launch_gemm_wgrad(g, st));
        g.sg = SgArgs{};
    }
    FQ_TRY(mark(events, 7, st));
    if (need_dxh) {
        // B7: A1 straight-through + unpermute-sum
        UnpermuteArgs ua{};
        ua.x = static_cast<const uint16_t*>(x);
        ua.dxh = dxh;
        ua.ids = topk_ids;
        ua.row_of = row_of;
        ua.dx = static_cast<uint16_t*>(dx);
        ua.rowpart = G->ds_a1 ? at<float>(workspace, lay.rowpart1) : nullptr;
        ua.T = T;
        ua.k = k;
        ua.H = H;
        ua.E = E;
        ua.a1 = ActQ{q.a1, P->s_a1};
        FQ_TRY(launch_unpermute_a1(ua, st));
        FQ_TRY(mark(events, 8, st));
        if (G->ds_a1) FQ_TRY(launch_segment_sum(ua.rowpart, offsets, E, unpermute_split((int)L->H), G->ds_a1, st));
    }

    if (!need_dxh) FQ_TRY(mark(events, 8, st));
    // B8: weight-scale gradients; formed in the GEMM epilogue (mode 1), summed
    // from its partials (mode 2), or from (W, dW^) by the fake-quant backward
    FQ_TRY(mark(events, 9, st));
    if (G->ds_w1 && m1 == 2)
        FQ_TRY(launch_sg_reduce(q.w1, at<float>(workspace, lay.sgp1), E, 2 * I, H, at<float>(workspace, lay.tws),
                                G->ds_w1, st));
    if (G->ds_w1 && m1 == 0) {
        TensorArgs ta{};
        ta.q = q.w1;
        ta.batch = E;
        ta.rows = 2 * I;
        ta.cols = H;
        ta.x = static_cast<const uint16_t*>(P->w1);
        ta.scale = P->s_w1;
        ta.tscale = P->t_w1;
        ta.gy = dw1;
        ta.gy_fp32 = 1;
        ta.gscale = G->ds_w1;
        ta.rowpart = at<float>(workspace, lay.tws);
        FQ_TRY(launch_tensor_bwd(ta, st));
    }
    FQ_TRY(mark(events, 10, st));
    if (G->ds_w2 && m2 == 2)
        FQ_TRY(launch_sg_reduce(q.w2, at<float>(workspace, lay.sgp2), E, H, I, at<float>(workspace, lay.tws),
                                G->ds_w2, st));
    if (G->ds_w2 && m2 == 0) {
        TensorArgs ta{};
        ta.q = q.w2;
        ta.batch = E;
        ta.rows = H;
        ta.cols = I;
        ta.x = static_cast<const uint16_t*>(P->w2);
        ta.scale = P->s_w2;
        ta.tscale = P->t_w2;
        ta.gy = dw2;
        ta.gy_fp32 = 1;
        ta.gscale = G->ds_w2;
        ta.rowpart = at<float>(workspace, lay.tws);
        FQ_TRY(launch_tensor_bwd(ta, st));
    }
    FQ_TRY(mark(events, FQ_BWD_STAGES, st));
    return FQ_OK;
}

int fq_adamw_defaults(fq_adamw_hparams* h) {
    if (!h) return FQ_E_INVALID;
    h->lr = 2.0e-4f;
    h->beta1 = 0.9f;
    h->beta2 = 0.95f;
    h->eps = 1.0e-8f;
    h->weight_decay = 0.0f;
    h->max_grad_norm = 1.0f;
    return FQ_OK;
}

size_t fq_scale_adamw_workspace_size(const fq_scale_param* params, int32_t nparams) {
    int64_t nb = 0;
    if (params && nparams > 0 && nparams <= FQ_MAX_SCALE_PARAMS)
        for (int i = 0; i < nparams; ++i) nb += adam_norm_blocks(params[i].count > 0 ? params[i].count : 0);
    return round_up((size_t)(nb > 0 ? nb : 1) * sizeof(double) + sizeof(double), 256);
}

// Scratch of fq_scale_adamw_noalloc: the norm pass's per-block partials and
// the clip factor.  Every block of the norm pass writes its own partial and
// the norm kernel writes the clip factor before the update reads it, so
// nothing here needs clearing between calls.  In host code the name is only
// a stand-in: kernels get the device address looked up per device below.
static __device__ __align__(256) double scratch[FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS + 1];

namespace {

// Validate one optimiser step and fill its launch arguments (all but the
// scratch pointers); *nb receives the norm pass's block count.
int adamw_args(const fq_scale_param* params, int32_t nparams, const fq_adamw_hparams* h, int64_t step,
               float* grad_norm, AdamArgs* out, int64_t* nb_out) {
    if (!params || !h || nparams < 1 || nparams > FQ_MAX_SCALE_PARAMS || step < 1) return FQ_E_INVALID;
    const float hv[6] = {h->lr, h->beta1, h->beta2, h->eps, h->weight_decay, h->max_grad_norm};
    for (float v : hv)
        if (!std::isfinite(v)) return FQ_E_INVALID;
    if (h->lr < 0 || h->beta1 < 0 || h->beta1 >= 1 || h->beta2 < 0 || h->beta2 >= 1 || h->eps <= 0 ||
        h->weight_decay < 0)
        return FQ_E_INVALID;
    AdamArgs a{};
    int64_t nb = 0;
    for (int i = 0; i < nparams; ++i) {
        const fq_scale_param& q = params[i];
        if (q.count < 0 || (q.proj != FQ_PROJ_POSITIVE && q.proj != FQ_PROJ_E4M3_BLOCK)) return FQ_E_INVALID;
        if (q.proj == FQ_PROJ_E4M3_BLOCK && (!q.tensor_scale || q.per_tensor < 1)) return FQ_E_INVALID;
        if (q.count > 0 && (!q.param || !q.grad || !q.exp_avg || !q.exp_avg_sq)) return FQ_E_INVALID;
        if (!aligned(q.param, 4) || !aligned(q.grad, 4) || !aligned(q.exp_avg, 4) || !aligned(q.exp_avg_sq, 4) ||
            !aligned(q.tensor_scale, 4))
            return FQ_E_ALIGN;
        const int64_t per = q.per_tensor > 0 ? q.per_tensor : 1;
        const bool vec = q.count % 4 == 0 && aligned(q.param, 16) && aligned(q.grad, 16) &&
                         aligned(q.exp_avg, 16) && aligned(q.exp_avg_sq, 16) &&
                         (q.proj != FQ_PROJ_E4M3_BLOCK || per % 4 == 0);
        a.prm[i] = AdamParam{q.param, q.grad, q.exp_avg, q.exp_avg_sq, q.count, nb, q.proj, vec ? 1 : 0,
                             q.tensor_scale, per};
        nb += adam_norm_blocks(q.count);
    }
    if (grad_norm && !aligned(grad_norm, 4)) return FQ_E_ALIGN;
    a.np = nparams;
    a.nb = nb;
    a.b1 = h->beta1;
    a.b2 = h->beta2;
    a.one_m_b1 = (float)(1.0 - (double)h->beta1);
    a.one_m_b2 = (float)(1.0 - (double)h->beta2);
    a.eps = h->eps;
    a.decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);
    const double bc1 = 1.0 - std::pow((double)h->beta1, (double)step);
    const double bc2 = 1.0 - std::pow((double)h->beta2, (double)step);
    a.step_size = (float)((double)h->lr / bc1);
    a.bc2_sqrt = (float)std::sqrt(bc2);
    a.max_norm = h->max_grad_norm;
    a.norm_out = grad_norm;
    *out = a;
    *nb_out = nb;
    return FQ_OK;
}

constexpr int64_t NOALLOC_ADAM_BLOCKS = FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS;
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
hipError_t scratch_on_current_device(double** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<double*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

int fq_scale_adamw(const fq_scale_param* params, int32_t nparams, const fq_adamw_hparams* h, int64_t step,
                   float* grad_norm, void* workspace, size_t workspace_bytes, void* stream) {
    AdamArgs a{};
    int64_t nb = 0;
    int s = adamw_args(params, nparams, h, step, grad_norm, &a, &nb);
    if (s != FQ_OK) return s;
    if (!workspace || !aligned(workspace, 8)) return workspace ? FQ_E_ALIGN : FQ_E_WORKSPACE;
    if (workspace_bytes < fq_scale_adamw_workspace_size(params, nparams)) return FQ_E_WORKSPACE;
    a.part = static_cast<double*>(workspace);
    a.clip = reinterpret_cast<float*>(static_cast<double*>(workspace) + a.nb);
    FQ_TRY(launch_scale_adamw(a, static_cast<hipStream_t>(stream)));
    return FQ_OK;
}

int fq_scale_adamw_noalloc(const fq_scale_param* params, int32_t nparams, const fq_adamw_hparams* h,
                           int64_t step, float* grad_norm, void* stream) {
    AdamArgs a{};
    int64_t nb = 0;
    int s = adamw_args(params, nparams, h, step, grad_norm, &a, &nb);
    if (s != FQ_OK) return s;
    if (nb > NOALLOC_ADAM_BLOCKS) return FQ_E_WORKSPACE;
    double* ptr = nullptr;
    FQ_TRY(scratch_on_current_device(&ptr));
    a.part = ptr;
    a.clip = reinterpret_cast<float*>(ptr + a.nb);
    FQ_TRY(launch_scale_adamw(a, static_cast<hipStream_t>(stream)));
    return FQ_OK;
}

size_t fq_distill_workspace_size(int64_t tokens) {
    return round_up((size_t)(tokens > 0 ? tokens : 1) * sizeof(float), 256);
}

int fq_distill_loss(const fq_distill_desc* d, int64_t tokens, int64_t vocab, const void* student_logits,
                    const void* teacher_logits, const float* teacher_topk_logits,
                    const int32_t* teacher_topk_ids, const int32_t* labels, float* loss, float* row_loss,
                    void* grad, void* workspace, size_t workspace_bytes, void* stream) {
    if (!d || !loss || (tokens > 0 && !student_logits)) return FQ_E_INVALID;   // no tokens: nothing is read
    if (d->type < FQ_DISTILL_KL || d->type > FQ_DISTILL_TOPK_KL) return FQ_E_INVALID;
    if (!std::isfinite(d->lm_weight) || !std::isfinite(d->distill_weight)) return FQ_E_INVALID;
    if (tokens < 0 || vocab < 8 || vocab % 8 || vocab >= ((int64_t)1 << 31)) return FQ_E_SHAPE;
    const bool topk = d->type == FQ_DISTILL_TOPK_KL;
    if (topk) {
        if (d->topk < 1 || d->topk > 64 || d->topk > vocab ||
            (tokens > 0 && (!teacher_topk_logits || !teacher_topk_ids)))
            return FQ_E_INVALID;
    } else if (d->topk != 0 || (tokens > 0 && !teacher_logits)) {
        return FQ_E_INVALID;
    }
    if (!aligned(student_logits, 16) || (!topk && !aligned(teacher_logits, 16)) || (grad && !aligned(grad, 16)) ||
        !aligned(loss, 4) || (row_loss && !aligned(row_loss, 4)) || (labels && !aligned(labels, 4)) ||
        (topk && (!aligned(teacher_topk_logits, 4) || !aligned(teacher_topk_ids, 4))))
        return FQ_E_ALIGN;
    if (!row_loss) {
        if (!workspace) return FQ_E_WORKSPACE;
        if (!aligned(workspace, 4)) return FQ_E_ALIGN;
        if (workspace_bytes < fq_distill_workspace_size(tokens)) return FQ_E_WORKSPACE;
    }
    DistillArgs a{};
    a.kind = d->type;
    a.T = tokens;
    a.V = vocab;
    a.zs = static_cast<const uint16_t*>(student_logits);
    a.zt = topk ? nullptr : static_cast<const uint16_t*>(teacher_logits);
    a.top_v = topk ? teacher_topk_logits : nullptr;
    a.top_i = topk ? teacher_topk_ids : nullptr;
    a.k = topk ? d->topk : 0;
    a.labels = labels;
    a.lm_w = d->lm_weight;
    a.dist_w = d->distill_weight;
    a.inv_T = tokens > 0 ? (float)(1.0 / (double)tokens) : 0.0f;
    a.row_loss = row_loss ? row_loss : static_cast<float*>(workspace);
    a.grad = static_cast<uint16_t*>(grad);
    FQ_TRY(launch_distill(a, loss, static_cast<hipStream_t>(stream)));
    return FQ_OK;
}

}  // extern "C"
