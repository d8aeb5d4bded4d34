// Routing and the element-wise stages of the grouped SwiGLU expert layer.
//
// The grouped-experts design of the nxmr.cn article on MCoreQAD (section 二.4)
// gathers the routed copies of the tokens expert by expert so that one grouped
// GEMM covers all experts; every matmul input is fake-quantised by its
// expert's activation quantiser on the way (section 二.3), and the router's
// ids and weights are unquantised inputs.
//
// Row order (a stable counting sort): experts ascending, and inside an expert
// the flat routing index t*k + j ascending.  All reductions below use fixed
// trees, so results are bitwise reproducible.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {

namespace {

constexpr int TPB = 256;
constexpr int RPB = TPB / WAVE;      // rows (tokens) per block, one per wave
constexpr int RB = 1024;             // routing elements per block

__device__ __forceinline__ int clamp_id(int id, int E) { return id < 0 ? 0 : (id >= E ? E - 1 : id); }
// routed-row indices read back from the routing tables, kept in [0, R)
__device__ __forceinline__ int64_t clamp_row(int64_t r, int64_t R) { return r < 0 ? 0 : (r >= R ? R - 1 : r); }

// The k routing slots of token t in one load: lane j < k holds slot j's
// expert, routed row and weight; slot j is then read with a wave-uniform
// readlane (k <= 64).
struct Slots {
    int e, row;
    float w;
};
__device__ __forceinline__ Slots load_slots(const int32_t* ids, const int32_t* row_of, const float* w, int64_t t,
                                            int k, int E, int64_t R, int lane) {
    Slots s{0, 0, 0.0f};
    if (lane < k) {
        const int64_t fi = t * k + lane;
        if (ids) s.e = clamp_id(ids[fi], E);
        s.row = (int)clamp_row(row_of[fi], R);
        if (w) s.w = w[fi];
    }
    return s;
}
__device__ __forceinline__ int slot_i(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ float slot_f(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// ------------------------------------------------------------------ routing --
// Per block of RB flat indices: histogram and the stable rank of each element
// among equal ids inside the block.  Equal ids inside a 64-element wave slice
// are found with one ballot per id bit; the wave slices of the block are
// ordered by a per-wave running histogram in LDS.
__global__ __launch_bounds__(TPB) void k_route_local(const int32_t* ids, int64_t R, int E,
                                                     int nbits, int32_t* hist, int32_t* local_rank) {
    extern __shared__ int32_t whist[];                    // [4][E]
    const int lane = threadIdx.x & (WAVE - 1);
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 4 * E; i += TPB) whist[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * RB + w * 256;
    int rk[4], idv[4];
#pragma unroll
    for (int sc = 0; sc < 4; ++sc) {
        const int64_t i = base + sc * WAVE + lane;
        const bool valid = i < R;
        const int id = valid ? clamp_id(ids[i], E) : 0;
        idv[sc] = id;
        uint64_t m = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (id >> bit) & 1;
            const uint64_t bal = __ballot(valid && on);
            m &= on ? bal : ~bal;
        }
        int before = 0;
        if (valid) {
            before = whist[w * E + id];
            rk[sc] = before + __popcll(m & ((1ull << lane) - 1ull));
        }
        // all lanes of this wave read the running count before the group's
        // lowest lane adds the group size (one instruction stream, in order)
        if (valid && lane == __ffsll((unsigned long long)m) - 1) whist[w * E + id] = before + __popcll(m);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += TPB) {
        const int s0 = whist[e], s1 = whist[E + e], s2 = whist[2 * E + e], s3 = whist[3 * E + e];
        whist[e] = 0;
        whist[E + e] = s0;
        whist[2 * E + e] = s0 + s1;
        whist[3 * E + e] = s0 + s1 + s2;
        hist[(int64_t)blockIdx.x * E + e] = s0 + s1 + s2 + s3;
    }
    __syncthreads();
#pragma unroll
    for (int sc = 0; sc < 4; ++sc) {
        const int64_t i = base + sc * WAVE + lane;
        if (i < R) local_rank[i] = whist[w * E + idv[sc]] + rk[sc];
    }
}

// One block: per-expert counts, block bases, offsets, the GEMM row-tile
// tables (heights 128 and 256) and the experts ordered by descending count
// (ties by id).
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* hist, int nblk, int E, int32_t* counts,
                                                     int32_t* offsets, TileTable t128, TileTable t256,
                                                     int32_t* order, int32_t* wg_list, int32_t* wg_cnt) {
    __shared__ int32_t s_cnt[1024];
    __shared__ int32_t s_ord[1024];
    __shared__ int32_t s_a[1024];
    __shared__ int32_t s_b[1024];
    __shared__ int32_t s_c[1024];
    __shared__ int32_t s_part[1024];
    const int e = threadIdx.x;
    // P threads per expert column: thread (ce, cj) = (t % E, t / E) owns the
    // contiguous run of blocks [b0, b1); its loads are independent, 8 at a time
    const int P = 1024 / E;
    const int ce = e % E, cj = e / E;
    const bool col = cj < P;
    const int chunk = (nblk + P - 1) / P;
    const int b0 = min(cj * chunk, nblk), b1 = col ? min(b0 + chunk, nblk) : b0;
    int part = 0;
    {
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            int h[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = hist[(int64_t)(b + u) * E + ce];
#pragma unroll
            for (int u = 0; u < 8; ++u) part += h[u];
        }
        for (; b < b1; ++b) part += hist[(int64_t)b * E + ce];
    }
    s_part[e] = part;
    __syncthreads();
    int running = 0;
    if (e < E)
        for (int j = 0; j < P; ++j) running += s_part[j * E + e];
    const int cnt = e < E ? running : 0;
    const int m1 = (cnt + 127) / 128, m2 = (cnt + 255) / 256;
    s_cnt[e] = cnt;
    s_a[e] = cnt;
    s_b[e] = m1;
    s_c[e] = m2;
    __syncthreads();
    // inclusive Hillis-Steele scans of counts and of both row-tile counts
    for (int d = 1; d < 1024; d <<= 1) {
        const int va = e >= d ? s_a[e - d] : 0;
        const int vb = e >= d ? s_b[e - d] : 0;
        const int vc = e >= d ? s_c[e - d] : 0;
        __syncthreads();
        s_a[e] += va;
        s_b[e] += vb;
        s_c[e] += vc;
        __syncthreads();
    }
    if (e < E) {
        const int off = s_a[e] - cnt;
        counts[e] = cnt;
        offsets[e] = off;
        if (e == E - 1) {
            offsets[E] = off + cnt;
            t128.num_tiles[0] = s_b[e];
            t256.num_tiles[0] = s_c[e];
        }
        int rank = 0;
        for (int o = 0; o < E; ++o) {
            const int c = s_cnt[o];
            rank += (c > cnt) || (c == cnt && o < e);
        }
        order[rank] = e;
        s_ord[rank] = e;
    }
    if (col) {
        // column ce's row-tile table entries i = cj, cj + P, ...
        const int cc = s_cnt[ce], off = s_a[ce] - cc;
        const int n1 = (cc + 127) / 128, n2 = (cc + 255) / 256;
        const int ts1 = s_b[ce] - n1, ts2 = s_c[ce] - n2;
        for (int i = cj; i < n1; i += P) {
            t128.tile_expert[ts1 + i] = ce;
            t128.tile_row0[ts1 + i] = off + i * 128;
        }
        for (int i = cj; i < n2; i += P) {
            t256.tile_expert[ts2 + i] = ce;
            t256.tile_row0[ts2 + i] = off + i * 256;
        }
        // each block's first row of expert ce: off + the exclusive prefix over
        // the earlier runs of the column, then over this run's blocks
        int acc = off;
        for (int j = 0; j < cj; ++j) acc += s_part[j * E + ce];
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            int h[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = hist[(int64_t)(b + u) * E + ce];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                hist[(int64_t)(b + u) * E + ce] = acc;
                acc += h[u];
            }
        }
        for (; b < b1; ++b) {
            const int h = hist[(int64_t)b * E + ce];
            hist[(int64_t)b * E + ce] = acc;
            acc += h;
        }
    }
    __syncthreads();
    // Weight-gradient work per XCD (each XCD has its own L2): experts in
    // descending count go to the least loaded XCD so far (ties: lowest XCD),
    // load = reduction steps of 64 rows + 2 for the epilogue.  One wave; lane
    // x < 8 keeps XCD x's load and list.  The experts come 64 at a time, one
    // per lane, and each step reads its expert and cost from a lane register.
    // (A form with the eight loads in scalar registers measured slower: about
    // 90 scalar instructions per step.)
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int load = 0, n = 0;
        for (int r0 = 0; r0 < E; r0 += 64) {
            const int ex_l = r0 + lane < E ? s_ord[r0 + lane] : 0;
            const int cost_l = (s_cnt[ex_l] + 63) / 64 + 2;
            const int nr = min(64, E - r0);
            for (int i = 0; i < nr; ++i) {
                const int ex = __builtin_amdgcn_readlane(ex_l, i);
                const int cost = __builtin_amdgcn_readlane(cost_l, i);
                // minimum over lanes 0-7 by DPP moves (no LDS round trip):
                // swap neighbours, swap pairs, then mirror the 8-lane half row
                int key = lane < 8 ? load * 8 + lane : 0x7FFFFFFF;
                key = min(key, __builtin_amdgcn_mov_dpp(key, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
                key = min(key, __builtin_amdgcn_mov_dpp(key, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
                key = min(key, __builtin_amdgcn_mov_dpp(key, 0x141, 0xF, 0xF, false));   // row_half_mirror
                if (lane == (key & 7)) {
                    wg_list[lane * E + n] = ex;
                    ++n;
                    load += cost;
                }
            }
        }
        if (lane < 8) wg_cnt[lane] = n;
    }
}

__global__ __launch_bounds__(TPB) void k_route_scatter(const int32_t* ids, int64_t R, int E,
                                                       const int32_t* hist, const int32_t* local_rank,
                                                       int32_t* row_of, int32_t* src_of, int32_t* row_expert) {
    const int64_t i0 = (int64_t)blockIdx.x * RB;
    for (int j = threadIdx.x; j < RB; j += TPB) {
        const int64_t i = i0 + j;
        if (i >= R) break;
        const int id = clamp_id(ids[i], E);
        const int row = hist[(int64_t)blockIdx.x * E + id] + local_rank[i];
        row_of[i] = row;
        if (row >= 0 && row < R) {
            src_of[row] = (int32_t)i;
            row_expert[row] = id;
        }
    }
}

// --------------------------------------------------------------- activation --
// The per-expert tensor scale the quantiser reads (0 where it has none):
// through the scalar cache when e is wave-uniform.
template <int KIND>
__device__ __forceinline__ float act_t(const ActQ& a, int e) {
    return (KIND == K_NVFP4 || (KIND != K_NONE && a.q.source != S_DYNAMIC)) ? sload(a.s, e) : 0.0f;
}

// Effective scale of an 8-element vector under the layer's activation
// quantiser, given its expert's tensor scale t = act_t(a, e).  `bm` is the
// vector's 16-block amax (NVFP4), `gm` its group amax (INT/FP8 per-group
// dynamic), `row_s` the dynamic per-row scale.
template <int KIND>
__device__ __forceinline__ float act_scale_t(const ActQ& a, float t, float bm, float gm, float row_s, float* dfac) {
    *dfac = 1.0f;
    if (KIND == K_NVFP4) {
        const float d6 = 6.0f * t;
        // fl32(bm / d6): Markstein's corrected quotient when every lane's d6
        // is normal, IEEE division otherwise.  Where the corrected form
        // overflows (a NaN) the quotient is far above 448, and fminf takes
        // 448 from both.
        float qd;
        if (__all(d6 >= 0x1p-120f && d6 <= 0x1p120f)) {
            const float inv = rcp_rn(d6);
            const float q0 = bm * inv;
            qd = __builtin_fmaf(__builtin_fmaf(-q0, d6, bm), inv, q0);
        } else {
            qd = bm / d6;
        }
        const float d = e4m3_round(fminf(qd, 448.0f));
        *dfac = d;
        return t * d;
    }
    if (a.q.source != S_DYNAMIC) return t;               // per-expert per-tensor scale
    if (a.q.gran == G_ROW) return row_s;
    return gm / a.q.qdiv;
}

// the same for expert e
template <int KIND>
__device__ __forceinline__ float act_scale(const ActQ& a, int e, float bm, float gm, float row_s, float* dfac) {
    return act_scale_t<KIND>(a, act_t<KIND>(a, e), bm, gm, row_s, dfac);
}

template <int KIND>
__device__ __forceinline__ void quant8(const float* f, float s, float qmin, float qmax, float* y) {
    quant_group<KIND, 8>(f, s, qmin, qmax, [&](int i, const Elem& e) { y[i] = e.q * s; });
}

// straight-through terms of 8 elements: sum g*c, and the pass mask applied to
// g (a dynamic quantiser passes every element)
template <int KIND, bool DYN>
__device__ __forceinline__ float ste8_(const float* f, const float* g, float s, float qmin, float qmax, float* gx) {
    float part = 0.0f;
    quant_group<KIND, 8>(f, s, qmin, qmax, [&](int i, const Elem& el) {
        part = __builtin_fmaf(g[i], ste_c(el, qmin, qmax), part);
        gx[i] = DYN ? g[i] : g[i] * (el.inside ? 1.0f : 0.0f);   // g * mask (signed zero)
    });
    return part;
}
// dyn is uniform (the quantiser's source): one branch, not a select per element
template <int KIND>
__device__ __forceinline__ float ste8(const float* f, const float* g, float s, float qmin, float qmax,
                                      bool dyn, float* gx) {
    return dyn ? ste8_<KIND, true>(f, g, s, qmin, qmax, gx) : ste8_<KIND, false>(f, g, s, qmin, qmax, gx);
}

__device__ __forceinline__ float amax8(const float* f) {
    float m = fabsf(f[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

// ------------------------------------------------------------ F2 permute+A1 --
// One wave per token: x[t] is read once, block / row statistics formed once,
// then each of its k routed copies is quantised with its expert's quantiser
// and written to its row.
// SPLIT waves per token, each on a contiguous 1/SPLIT of the row, unless the
// quantiser's scale is a whole-row statistic (dynamic per row).
template <int KIND, int NV, int SPLIT>
__global__ __launch_bounds__(TPB) void k_permute_a1(PermuteArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nvec = (a.H >> 3) / SPLIT;         // vectors of 8 in this wave's part of the row
    const float qmin = a.a1.q.qmin, qmax = a.a1.q.qmax;
    const int gl = a.a1.q.group >> 3;
    const bool indep = KIND != K_NONE && KIND != K_NVFP4 && a.a1.q.source == S_DYNAMIC;
    for (int64_t w = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6); w < a.T * SPLIT;
         w += (int64_t)gridDim.x * RPB) {
        const int64_t t = w / SPLIT;
        const int64_t c0 = (w - t * SPLIT) * nvec * 8;  // first column of this part
        uint4 xv[NV];
        float bm[NV];
        float rm = 0.0f;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int v = lane + c * WAVE;
            xv[c] = v < nvec ? reinterpret_cast<const uint4*>(a.x + t * a.H + c0)[v] : make_uint4(0, 0, 0, 0);
            float f[8];
            unpack8(xv[c], f);
            const float m = amax8(f);
            rm = fmaxf(rm, m);
            if (KIND == K_NVFP4) bm[c] = fmaxf(m, __shfl_xor(m, 1));
            else if (KIND != K_NONE && a.a1.q.gran == G_GROUP) bm[c] = group_max(m, gl);
            else bm[c] = 0.0f;
        }
        float row_s = 0.0f;
        if (KIND != K_NONE && KIND != K_NVFP4 && a.a1.q.gran == G_ROW && a.a1.q.source == S_DYNAMIC)
            row_s = wave_max(rm) / a.a1.q.qdiv;
        uint4 qv[NV];
        if (indep) {                                    // same quantised row for every expert
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                float f[8], y[8], dfac;
                unpack8(xv[c], f);
                quant8<KIND>(f, act_scale<KIND>(a.a1, 0, bm[c], bm[c], row_s, &dfac), qmin, qmax, y);
                qv[c] = pack8(y);
            }
        }
        const Slots sl = load_slots(a.ids, a.row_of, nullptr, t, a.k, a.E, a.T * a.k, lane);
        for (int j = 0; j < a.k; ++j) {
            const int e = slot_i(sl.e, j);
            const int64_t row = slot_i(sl.row, j);
            uint4* dst = reinterpret_cast<uint4*>(a.xhat + row * a.H + c0);
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                if (v >= nvec) continue;
                if (KIND == K_NONE) {
                    dst[v] = xv[c];
                } else if (indep) {
                    dst[v] = qv[c];
                } else {
                    float f[8], y[8], dfac;
                    unpack8(xv[c], f);
                    quant8<KIND>(f, act_scale<KIND>(a.a1, e, bm[c], bm[c], row_s, &dfac), qmin, qmax, y);
                    dst[v] = pack8(y);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ SiLU ----
// silu(g) = g / (1 + e^-g) in fp32, within (8 + 2|g|) 2^-24 of the exact value
// (relative; results below 2^-126 within that plus (1 + |g|) 2^-149).
// e^-|g| = 2^y, y = -|g| log2(e) clamped at -200 (2^-200 is 0 in fp32):
// 2^y = 2^rint(y) * P(y - rint(y)), P the degree-7 Taylor polynomial of 2^f
// (coefficients (ln 2)^i / i!, rounded to fp32), Horner with one fused
// multiply-add per degree; the 2|g| term is the rounding of y.
__device__ __forceinline__ float exp2_taylor(float y) {
    const float n = rintf(y);
    const float f = y - n;
    float p = 0x1.ffcbfcp-17f;
    p = __builtin_fmaf(p, f, 0x1.430912p-13f);
    p = __builtin_fmaf(p, f, 0x1.5d87fep-10f);
    p = __builtin_fmaf(p, f, 0x1.3b2ab6p-7f);
    p = __builtin_fmaf(p, f, 0x1.c6b08ep-5f);
    p = __builtin_fmaf(p, f, 0x1.ebfbe0p-3f);
    p = __builtin_fmaf(p, f, 0x1.62e430p-1f);
    p = __builtin_fmaf(p, f, 1.0f);
    return ldexpf(p, (int)n);
}

// silu(g) and sigmoid(g), as the forward and the backward both form them,
// without branches and without overflow: with e = e^-|g| in [0, 1] and
// den = 1 + e in [1, 2],
//     g >= 0:  silu = g / den,      sigmoid = 1 / den
//     g <  0:  silu = g e / den,    sigmoid = e / den
// (both are g / (1 + e^-g)).  The quotient is Markstein's correction of
// num RN(1/den) (the rounded quotient while it is normal): where e rounds
// away (den = 1) silu is g exactly, as the exact value rounds; the sign is
// g's, so silu(-0) = -0.
__device__ __forceinline__ float silu_sig(float g, float* sig) {
    const float e = exp2_taylor(fmaxf(-fabsf(g) * 0x1.715476p+0f, -200.0f));
    const float den = 1.0f + e;
    const float inv = rcp_rn(den);
    const float sel = g < 0.0f ? e : 1.0f;
    const float num = g * sel;
    const float q0 = num * inv;
    const float r = __builtin_fmaf(__builtin_fmaf(-q0, den, num), inv, q0);
    *sig = sel * inv;
    return __builtin_copysignf(r, g);
}

// ------------------------------------------------------------- F5 SwiGLU+A2 --
// RW rows per wave: with RW = 2 (used when a row has 32 mod 64 vectors of 8)
// the wave's vectors u = lane + 64 c run over both rows, row u / nvec, so no
// lane idles on a half-filled last pass.  16-blocks and quantiser groups never
// straddle the two rows (nvec is a multiple of the group's vector count).
template <int KIND, int NV, int RW>
__global__ __launch_bounds__(TPB) void k_swiglu_a2(SwigluArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nvec = a.I >> 3;
    const float qmin = a.a2.q.qmin, qmax = a.a2.q.qmax;
    const int gl = a.a2.q.group >> 3;
    for (int64_t r0 = ((int64_t)blockIdx.x * RPB + (threadIdx.x >> 6)) * RW; r0 < a.R;
         r0 += (int64_t)gridDim.x * RPB * RW) {
        int ex[RW];
        float tx[RW];                                    // the rows' tensor scales, read before any store
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            ex[i] = r0 + i < a.R ? clamp_id(a.row_expert[r0 + i], a.E) : 0;
            tx[i] = act_t<KIND>(a.a2, ex[i]);
        }
        uint4 hv[NV];
        float bm[NV];
        float rm[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) rm[i] = 0.0f;
        // every vector's inputs first, then one wait
        uint4 zg[NV], zu[NV];
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int u = lane + c * WAVE;
            const int ri = (RW == 2 && u >= nvec) ? 1 : 0;
            const int v = u - ri * nvec;
            zg[c] = zu[c] = make_uint4(0, 0, 0, 0);
            if (u < RW * nvec && r0 + ri < a.R) {
                const uint4* zr = reinterpret_cast<const uint4*>(a.z1 + (r0 + ri) * 2 * (int64_t)a.I);
                zg[c] = zr[v];
                zu[c] = zr[v + nvec];
            }
        }
        vm_wait<0>();
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int u = lane + c * WAVE;
            const int ri = (RW == 2 && u >= nvec) ? 1 : 0;
            float h[8];
            if (u < RW * nvec && r0 + ri < a.R) {
                float g[8], uu[8];
                unpack8(zg[c], g);
                unpack8(zu[c], uu);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float sig;
                    h[i] = silu_sig(g[i], &sig) * uu[i];
                }
                hv[c] = pack8(h);
                unpack8(hv[c], h);                       // h as stored (bf16)
            } else {
                hv[c] = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) h[i] = 0.0f;
            }
            const float m = amax8(h);
#pragma unroll
            for (int i = 0; i < RW; ++i)
                if (ri == i) rm[i] = fmaxf(rm[i], m);
            if (KIND == K_NVFP4) bm[c] = fmaxf(m, __shfl_xor(m, 1));
            else if (KIND != K_NONE && a.a2.q.gran == G_GROUP) bm[c] = group_max(m, gl);
            else bm[c] = 0.0f;
        }
        float row_s[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            row_s[i] = 0.0f;
            if (KIND != K_NONE && KIND != K_NVFP4 && a.a2.q.gran == G_ROW && a.a2.q.source == S_DYNAMIC)
                row_s[i] = wave_max(rm[i]) / a.a2.q.qdiv;
        }
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int u = lane + c * WAVE;
            const int ri = (RW == 2 && u >= nvec) ? 1 : 0;
            const int v = u - ri * nvec;
            if (u >= RW * nvec || r0 + ri >= a.R) continue;
            uint4* dst = reinterpret_cast<uint4*>(a.hhat + (r0 + ri) * a.I);
            if (KIND == K_NONE) {
                dst[v] = hv[c];
            } else {
                float h[8], y[8], dfac;
                unpack8(hv[c], h);
                const float te = RW == 2 && ri ? tx[RW - 1] : tx[0];
                const float rs = RW == 2 && ri ? row_s[RW - 1] : row_s[0];
                quant8<KIND>(h, act_scale_t<KIND>(a.a2, te, bm[c], bm[c], rs, &dfac), qmin, qmax, y);
                dst[v] = pack8(y);
            }
        }
    }
}

// ------------------------------------------------------------- F7 combine ---
template <int NV>
__global__ __launch_bounds__(TPB) void k_combine(CombineArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nvec = a.H >> 3;
    for (int64_t t = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6); t < a.T; t += (int64_t)gridDim.x * RPB) {
        const Slots sl = load_slots(nullptr, a.row_of, a.w, t, a.k, 1, a.T * a.k, lane);
        float acc[NV][8];
#pragma unroll
        for (int c = 0; c < NV; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
        // row j+1 is loaded while row j is accumulated
        uint4 cur[NV], nxt[NV] = {};
        auto load = [&](int j, uint4* dst) {
            const uint4* src = reinterpret_cast<const uint4*>(a.yr + (int64_t)slot_i(sl.row, j) * a.H);
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                dst[c] = v < nvec ? src[v] : make_uint4(0, 0, 0, 0);
            }
        };
        load(0, cur);
        for (int j = 0; j < a.k; ++j) {
            if (j + 1 < a.k) load(j + 1, nxt);
            const float w = slot_f(sl.w, j);
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                float f[8];
                unpack8(cur[c], f);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[c][i] = acc[c][i] + w * f[i];
                cur[c] = nxt[c];
            }
        }
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int v = lane + c * WAVE;
            if (v < nvec) reinterpret_cast<uint4*>(a.y + t * a.H)[v] = pack8(acc[c]);
        }
    }
}

// ------------------------------------------------------------- B1 permute dY --
constexpr int KU = 8;                   // top-k of the unrolled path
template <int NV>
__global__ __launch_bounds__(TPB) void k_permute_dy(PermuteDyArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nvec = a.H >> 3;
    for (int64_t t = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6); t < a.T; t += (int64_t)gridDim.x * RPB) {
        const Slots sl = load_slots(nullptr, a.row_of, a.w, t, a.k, 1, a.T * a.k, lane);
        float d[NV][8];
        if (nvec == NV * WAVE && a.dw && a.k == KU) {
            // Every lane holds NV whole vectors and there are KU copies:
            // straight-line code in which a wait names only the row it needs.
            // Y_r row j+1 is loaded while row j is reduced, and it is issued
            // before row j's stores, so no wait is for a store.
            const uint4* dyt = reinterpret_cast<const uint4*>(a.dy + t * a.H);
            uint4 dv[NV];
#pragma unroll
            for (int c = 0; c < NV; ++c) dv[c] = dyt[lane + c * WAVE];
            uint4 yb[2][NV];
            auto load_y = [&](int j, uint4* dst) {
                const uint4* src = reinterpret_cast<const uint4*>(a.yr + (int64_t)slot_i(sl.row, j) * a.H);
#pragma unroll
                for (int c = 0; c < NV; ++c) dst[c] = src[lane + c * WAVE];
            };
            load_y(0, yb[0]);
#pragma unroll
            for (int c = 0; c < NV; ++c) unpack8(dv[c], d[c]);
            float dwl = 0.0f;                            // lane j: copy j's d topk_w
#pragma unroll
            for (int j = 0; j < KU; ++j) {
                if (j + 1 < KU) load_y(j + 1, yb[(j + 1) & 1]);
                const float w = slot_f(sl.w, j);
                const int64_t row = slot_i(sl.row, j);
                uint4* dst = reinterpret_cast<uint4*>(a.dyr + row * a.H);
                float part = 0.0f;
#pragma unroll
                for (int c = 0; c < NV; ++c) {
                    float o[8], yv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[i] = w * d[c][i];
                    dst[lane + c * WAVE] = pack8(o);
                    unpack8(yb[j & 1][c], yv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) part = __builtin_fmaf(d[c][i], yv[i], part);
                }
                part = wave_sum(part);
                dwl = lane == j ? part : dwl;
            }
            if (lane < KU) a.dw[t * a.k + lane] = dwl;
            continue;
        }
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int v = lane + c * WAVE;
            if (v < nvec) unpack8(reinterpret_cast<const uint4*>(a.dy + t * a.H)[v], d[c]);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) d[c][i] = 0.0f;
        }
        // with d topk_w: Y_r row j+1 is loaded while row j is reduced
        uint4 cur[NV], nxt[NV] = {};
        auto load = [&](int j, uint4* dst) {
            const uint4* src = reinterpret_cast<const uint4*>(a.yr + (int64_t)slot_i(sl.row, j) * a.H);
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                dst[c] = v < nvec ? src[v] : make_uint4(0, 0, 0, 0);
            }
        };
        if (a.dw) load(0, cur);
        for (int j = 0; j < a.k; ++j) {
            if (a.dw && j + 1 < a.k) load(j + 1, nxt);
            const float w = slot_f(sl.w, j);
            const int64_t row = slot_i(sl.row, j);
            float part = 0.0f;
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = w * d[c][i];
                if (v < nvec) reinterpret_cast<uint4*>(a.dyr + row * a.H)[v] = pack8(o);
                if (a.dw) {
                    float yv[8];
                    unpack8(cur[c], yv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) part = __builtin_fmaf(d[c][i], yv[i], part);
                    cur[c] = nxt[c];
                }
            }
            if (a.dw) {
                part = wave_sum(part);
                if (lane == 0) a.dw[t * a.k + j] = part;
            }
        }
    }
}

// --------------------------------------------- B4 A2 backward + SwiGLU backward --
// RW rows per wave as in the forward above.
template <int KIND, int RW>
__global__ __launch_bounds__(TPB) void k_swiglu_bwd(SwigluBwdArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nvec = a.I >> 3;
    const float qmin = a.a2.q.qmin, qmax = a.a2.q.qmax;
    const bool dyn = a.a2.q.source == S_DYNAMIC;
    // NVFP4 (dynamic blocks, learnable tensor scale) and per-tensor INT/FP8
    // need the forward's codec terms; per-row/group dynamic quantisers pass
    // the gradient straight and own no parameter.
    const bool recompute = KIND == K_NVFP4 || (KIND != K_NONE && !dyn);
    // passes of the wave over its rows
    const int npass = (RW * nvec + WAVE - 1) / WAVE;
    for (int64_t r0 = ((int64_t)blockIdx.x * RPB + (threadIdx.x >> 6)) * RW; r0 < a.R;
         r0 += (int64_t)gridDim.x * RPB * RW) {
        int ex[RW];
        float tx[RW], part_row[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            ex[i] = r0 + i < a.R ? clamp_id(a.row_expert[r0 + i], a.E) : 0;
            tx[i] = recompute ? act_t<KIND>(a.a2, ex[i]) : 0.0f;
            part_row[i] = 0.0f;
        }
        // pass p: this lane's vector (row r0 + ri, vector v) and its inputs
        auto load_pass = [&](int p, uint4& zg, uint4& zu, uint4& zd) {
            const int uf = p * WAVE + lane;
            const int ri = (RW == 2 && uf >= nvec) ? 1 : 0;
            const int v = uf - ri * nvec;
            const int64_t r = r0 + ri;
            if (uf < RW * nvec && r < a.R) {
                const uint4* zr = reinterpret_cast<const uint4*>(a.z1 + r * 2 * (int64_t)a.I);
                zg = zr[v];
                zu = zr[v + nvec];
                zd = reinterpret_cast<const uint4*>(a.dhh + r * a.I)[v];
            } else {
                zg = zu = zd = make_uint4(0, 0, 0, 0);
            }
        };
        auto run_pass = [&](int p, const uint4& zg, const uint4& zu, const uint4& zd) {
            const int uf = p * WAVE + lane;
            const int ri = (RW == 2 && uf >= nvec) ? 1 : 0;
            const int v = uf - ri * nvec;
            const int64_t r = r0 + ri;
            const bool act = uf < RW * nvec && r < a.R;
            uint4* out = reinterpret_cast<uint4*>(a.dz1 + r * 2 * (int64_t)a.I);
            float g[8], u[8], dh[8], sg[8], h[8];
            unpack8(zg, g);
            unpack8(zu, u);
            unpack8(zd, dh);
            // silu and sigmoid as the forward forms them
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = silu_sig(g[i], &sg[i]) * u[i];
            if (recompute) {
                float hq[8];
                unpack8(pack8(h), hq);                       // h as the forward stored it
                float bm = 0.0f;
                if (KIND == K_NVFP4) {
                    const float m = amax8(hq);
                    bm = fmaxf(m, __shfl_xor(m, 1));
                }
                float dfac;
                const float te = RW == 2 && ri ? tx[RW - 1] : tx[0];
                const float s = act_scale_t<KIND>(a.a2, te, bm, bm, 0.0f, &dfac);
                float gx[8];
                const float part = ste8<KIND>(hq, dh, s, qmin, qmax, dyn, gx);
                if (act) {
#pragma unroll
                    for (int i = 0; i < RW; ++i)
                        if (ri == i) part_row[i] = __builtin_fmaf(part, dfac, part_row[i]);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) dh[i] = gx[i];
            }
            if (act) {
                float dg[8], du[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float s = sg[i];
                    const float silu = g[i] * s;
                    dg[i] = dh[i] * u[i] * (s * (1.0f + g[i] * (1.0f - s)));
                    du[i] = dh[i] * silu;
                }
                out[v] = pack8(dg);
                out[v + nvec] = pack8(du);
            }
        };
        for (int p = 0; p < npass; ++p) {
            uint4 zg, zu, zd;
            load_pass(p, zg, zu, zd);
            run_pass(p, zg, zu, zd);
        }
        if (a.rowpart) {
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                const float tot = wave_sum(part_row[i]);
                if (lane == 0 && r0 + i < a.R) a.rowpart[r0 + i] = tot;
            }
        }
    }
}

// ------------------------------------------- B7 A1 backward + unpermute-sum --
// SPLIT waves per token, each on a contiguous 1/SPLIT of the row: the recomputed
// codec terms depend only on 16-blocks or a per-expert scale, never on the
// whole row, and parts of a row keep the wave's registers (and occupancy) in
// bounds; quarter rows (one vector per lane at H = 2048) double the waves in
// flight over half rows.  The per-row partial of ds_a1 is then SPLIT
// partials, rowpart[row SPLIT + part].
template <int KIND, int NV, int SPLIT>
__global__ __launch_bounds__(TPB) void k_unpermute_a1(UnpermuteArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nvl = (a.H >> 3) / SPLIT;          // vectors of 8 in this wave's part of the row
    const float qmin = a.a1.q.qmin, qmax = a.a1.q.qmax;
    const bool dyn = a.a1.q.source == S_DYNAMIC;
    const bool recompute = KIND == K_NVFP4 || (KIND != K_NONE && !dyn);
    for (int64_t w = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6); w < a.T * SPLIT;
         w += (int64_t)gridDim.x * RPB) {
        const int64_t t = w / SPLIT;
        const int hf = (int)(w - t * SPLIT);
        const int nvec = nvl;                    // the loops below see only this part
        const uint16_t* xrow = a.x + t * a.H + hf * nvl * 8;
        uint4 xv[NV];
        float bm[NV];
        if (recompute) {
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                xv[c] = v < nvec ? reinterpret_cast<const uint4*>(xrow)[v] : make_uint4(0, 0, 0, 0);
                float f[8];
                unpack8(xv[c], f);
                const float m = amax8(f);
                bm[c] = KIND == K_NVFP4 ? fmaxf(m, __shfl_xor(m, 1)) : 0.0f;
            }
        }
        float acc[NV][8];
#pragma unroll
        for (int c = 0; c < NV; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
        const Slots sl = load_slots(a.ids, a.row_of, nullptr, t, a.k, a.E, a.T * a.k, lane);
        float rp = 0.0f;
        // copy j's part of the routed gradient, reduced into acc; dv: its
        // vectors, already loaded
        auto reduce_copy = [&](int j, const uint4* dv) {
            const int e = slot_i(sl.e, j);
            float part_row = 0.0f;
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                if (v >= nvec) continue;
                float d[8];
                unpack8(dv[c], d);
                if (recompute) {
                    float f[8], gx[8], dfac;
                    unpack8(xv[c], f);
                    const float s = act_scale<KIND>(a.a1, e, bm[c], bm[c], 0.0f, &dfac);
                    const float part = ste8<KIND>(f, d, s, qmin, qmax, dyn, gx);
                    part_row = __builtin_fmaf(part, dfac, part_row);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[c][i] = acc[c][i] + gx[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[c][i] = acc[c][i] + d[i];
                }
            }
            if (a.rowpart) {
                const float tot = wave_sum(part_row);
                rp = lane == j ? tot : rp;
            }
        };
        auto copy_src = [&](int j) {
            return reinterpret_cast<const uint4*>(a.dxh + (int64_t)slot_i(sl.row, j) * a.H + hf * nvl * 8);
        };
        bool done = false;
        if constexpr (NV == 1) {
            if (a.k == KU && nvec == WAVE) {
                // straight-line top-KU: copy j+1's load goes out before copy j
                // is reduced, so each wait names one load (no stores between)
                uint4 db[2][1];
                db[0][0] = copy_src(0)[lane];
#pragma unroll
                for (int j = 0; j < KU; ++j) {
                    if (j + 1 < KU) db[(j + 1) & 1][0] = copy_src(j + 1)[lane];
                    reduce_copy(j, db[j & 1]);
                }
                done = true;
            }
        }
        if (!done) {
            for (int j = 0; j < a.k; ++j) {
                const uint4* src = copy_src(j);
                uint4 dv[NV];
#pragma unroll
                for (int c = 0; c < NV; ++c) {
                    const int v = lane + c * WAVE;
                    dv[c] = v < nvec ? src[v] : make_uint4(0, 0, 0, 0);
                }
                reduce_copy(j, dv);
            }
        }
        // lane j holds copy j's row and partial: one store after the loop, so
        // no load above waits behind a store
        if (a.rowpart && lane < a.k) a.rowpart[(int64_t)sl.row * SPLIT + hf] = rp;
        if (a.dx) {
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const int v = lane + c * WAVE;
                if (v < nvec) reinterpret_cast<uint4*>(a.dx + t * a.H + hf * nvl * 8)[v] = pack8(acc[c]);
            }
        }
    }
}

// ---------------------------------------------------- per-expert segment sum --
// One block per expert; each thread adds four independent loads per step (in a
// fixed order), then the waves' sums are combined in wave order: the result
// depends only on the segment's length, never on timing.
constexpr int SEG_TPB = 1024;
__global__ __launch_bounds__(SEG_TPB) void k_segment_sum(const float* rowpart, const int32_t* offsets, int per,
                                                      float* out) {
    __shared__ float red[SEG_TPB / WAVE];
    const int e = blockIdx.x;
    const int64_t lo = (int64_t)offsets[e] * per, hi = (int64_t)offsets[e + 1] * per;
    float acc = 0.0f;
    int64_t r = lo + threadIdx.x;
    for (; r + 3 * SEG_TPB < hi; r += 4 * SEG_TPB) {
        const float a0 = rowpart[r], a1 = rowpart[r + SEG_TPB];
        const float a2 = rowpart[r + 2 * SEG_TPB], a3 = rowpart[r + 3 * SEG_TPB];
        acc += (a0 + a1) + (a2 + a3);
    }
    for (; r < hi; r += SEG_TPB) acc += rowpart[r];
    acc = wave_sum(acc);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < SEG_TPB / WAVE; ++w) t += red[w];
        out[e] = t;
    }
}

unsigned grid_waves(int64_t n) {
    int64_t g = (n + RPB - 1) / RPB;
    if (g < 1) g = 1;
    if (g > (1 << 20)) g = 1 << 20;
    return (unsigned)g;
}

int nv_for(int H) { return H <= 1024 ? 2 : H <= 2048 ? 4 : H <= 4096 ? 8 : 16; }

}  // namespace

int64_t route_blocks(int64_t R) { return (R + RB - 1) / RB; }
int64_t max_mtiles(int64_t R, int E, int height) { return (R + height - 1) / height + E; }

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
    if (a.E > 1024) return hipErrorInvalidValue;
    const int64_t nblk = route_blocks(a.R);
    int nbits = 0;
    while ((1 << nbits) < a.E) ++nbits;
    if (nblk > 0) {
        hipLaunchKernelGGL(k_route_local, dim3((unsigned)nblk), dim3(TPB), 4 * a.E * sizeof(int32_t), st,
                           a.ids, a.R, a.E, nbits, a.hist, a.local_rank);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, st, a.hist, (int)nblk, a.E, a.counts,
                       a.offsets, a.tables[0], a.tables[1], a.order, a.wg_list, a.wg_cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nblk == 0) return err;
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)nblk), dim3(TPB), 0, st, a.ids, a.R, a.E, a.hist,
                       a.local_rank, a.row_of, a.src_of, a.row_expert);
    return hipGetLastError();
}

#define FQ_NV_SWITCH(NVV, KERNEL, KIND, GRID, ARGS)                                         \
    switch (NVV) {                                                                           \
    case 2: hipLaunchKernelGGL((KERNEL<KIND, 2>), GRID, dim3(TPB), 0, st, ARGS); break;      \
    case 4: hipLaunchKernelGGL((KERNEL<KIND, 4>), GRID, dim3(TPB), 0, st, ARGS); break;      \
    case 8: hipLaunchKernelGGL((KERNEL<KIND, 8>), GRID, dim3(TPB), 0, st, ARGS); break;      \
    default: hipLaunchKernelGGL((KERNEL<KIND, 16>), GRID, dim3(TPB), 0, st, ARGS); break;    \
    }

#define FQ_KIND_NV_SWITCH(KINDV, NVV, KERNEL, GRID, ARGS)                                   \
    switch (KINDV) {                                                                         \
    case K_NONE: FQ_NV_SWITCH(NVV, KERNEL, K_NONE, GRID, ARGS); break;                       \
    case K_NVFP4: FQ_NV_SWITCH(NVV, KERNEL, K_NVFP4, GRID, ARGS); break;                     \
    case K_INT: FQ_NV_SWITCH(NVV, KERNEL, K_INT, GRID, ARGS); break;                         \
    default: FQ_NV_SWITCH(NVV, KERNEL, K_FP8, GRID, ARGS); break;                            \
    }

hipError_t launch_permute_a1(const PermuteArgs& a, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    const bool row_stat = a.a1.q.kind != K_NONE && a.a1.q.kind != K_NVFP4 && a.a1.q.gran == G_ROW &&
                          a.a1.q.source == S_DYNAMIC;
    // half rows per wave (quarter rows measured slower here than in the backward)
    const int split = row_stat ? 1 : ((a.H >> 3) % 128 == 0 && (a.H >> 3) >= 256 ? 2 : 1);
    const dim3 grid(grid_waves(a.T * split));
    const int nv = nv_for(a.H / split);
#define FQ_PERM(KIND)                                                                                   \
    if (split == 2) {                                                                                   \
        switch (nv) {                                                                                   \
        case 2: hipLaunchKernelGGL((k_permute_a1<KIND, 2, 2>), grid, dim3(TPB), 0, st, a); break;       \
        case 4: hipLaunchKernelGGL((k_permute_a1<KIND, 4, 2>), grid, dim3(TPB), 0, st, a); break;       \
        default: hipLaunchKernelGGL((k_permute_a1<KIND, 8, 2>), grid, dim3(TPB), 0, st, a); break;      \
        }                                                                                               \
    } else {                                                                                            \
        switch (nv) {                                                                                   \
        case 2: hipLaunchKernelGGL((k_permute_a1<KIND, 2, 1>), grid, dim3(TPB), 0, st, a); break;       \
        case 4: hipLaunchKernelGGL((k_permute_a1<KIND, 4, 1>), grid, dim3(TPB), 0, st, a); break;       \
        case 8: hipLaunchKernelGGL((k_permute_a1<KIND, 8, 1>), grid, dim3(TPB), 0, st, a); break;       \
        default: hipLaunchKernelGGL((k_permute_a1<KIND, 16, 1>), grid, dim3(TPB), 0, st, a); break;    \
        }                                                                                               \
    }
    switch (a.a1.q.kind) {
    case K_NONE: FQ_PERM(K_NONE); break;
    case K_NVFP4: FQ_PERM(K_NVFP4); break;
    case K_INT: FQ_PERM(K_INT); break;
    default: FQ_PERM(K_FP8); break;
    }
#undef FQ_PERM
    return hipGetLastError();
}

// two rows per wave when a row is 32, 96, 160 or 224 vectors of 8 (then both
// rows fill 1, 3, 5 or 7 whole passes of the wave)
static int paired_nv(int I) {
    const int nvec = I >> 3;
    return (nvec % 64 == 32 && nvec <= 224) ? 2 * nvec / 64 : 0;
}

#define FQ_SWIGLU_PAIRED(KIND, NVV, GRID)                                                          \
    switch (NVV) {                                                                                  \
    case 1: hipLaunchKernelGGL((k_swiglu_a2<KIND, 1, 2>), GRID, dim3(TPB), 0, st, a); break;        \
    case 3: hipLaunchKernelGGL((k_swiglu_a2<KIND, 3, 2>), GRID, dim3(TPB), 0, st, a); break;        \
    case 5: hipLaunchKernelGGL((k_swiglu_a2<KIND, 5, 2>), GRID, dim3(TPB), 0, st, a); break;        \
    default: hipLaunchKernelGGL((k_swiglu_a2<KIND, 7, 2>), GRID, dim3(TPB), 0, st, a); break;       \
    }
#define FQ_SWIGLU_SINGLE(KIND, NVV, GRID)                                                          \
    switch (NVV) {                                                                                  \
    case 2: hipLaunchKernelGGL((k_swiglu_a2<KIND, 2, 1>), GRID, dim3(TPB), 0, st, a); break;        \
    case 4: hipLaunchKernelGGL((k_swiglu_a2<KIND, 4, 1>), GRID, dim3(TPB), 0, st, a); break;        \
    case 8: hipLaunchKernelGGL((k_swiglu_a2<KIND, 8, 1>), GRID, dim3(TPB), 0, st, a); break;        \
    default: hipLaunchKernelGGL((k_swiglu_a2<KIND, 16, 1>), GRID, dim3(TPB), 0, st, a); break;      \
    }

hipError_t launch_swiglu_a2(const SwigluArgs& a, hipStream_t st) {
    if (a.R == 0) return hipSuccess;
    const int pnv = paired_nv(a.I);
    const dim3 grid(grid_waves(pnv ? (a.R + 1) / 2 : a.R));
#define FQ_SWIGLU_FWD(KIND)                                                                         \
    if (pnv) { FQ_SWIGLU_PAIRED(KIND, pnv, grid) }                                                  \
    else { FQ_SWIGLU_SINGLE(KIND, nv_for(a.I), grid) }
    switch (a.a2.q.kind) {
    case K_NONE: FQ_SWIGLU_FWD(K_NONE); break;
    case K_NVFP4: FQ_SWIGLU_FWD(K_NVFP4); break;
    case K_INT: FQ_SWIGLU_FWD(K_INT); break;
    default: FQ_SWIGLU_FWD(K_FP8); break;
    }
#undef FQ_SWIGLU_FWD
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    const dim3 grid(grid_waves(a.T));
    switch (nv_for(a.H)) {
    case 2: hipLaunchKernelGGL(k_combine<2>, grid, dim3(TPB), 0, st, a); break;
    case 4: hipLaunchKernelGGL(k_combine<4>, grid, dim3(TPB), 0, st, a); break;
    case 8: hipLaunchKernelGGL(k_combine<8>, grid, dim3(TPB), 0, st, a); break;
    default: hipLaunchKernelGGL(k_combine<16>, grid, dim3(TPB), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_permute_dy(const PermuteDyArgs& a, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    const dim3 grid(grid_waves(a.T));
    switch (nv_for(a.H)) {
    case 2: hipLaunchKernelGGL(k_permute_dy<2>, grid, dim3(TPB), 0, st, a); break;
    case 4: hipLaunchKernelGGL(k_permute_dy<4>, grid, dim3(TPB), 0, st, a); break;
    case 8: hipLaunchKernelGGL(k_permute_dy<8>, grid, dim3(TPB), 0, st, a); break;
    default: hipLaunchKernelGGL(k_permute_dy<16>, grid, dim3(TPB), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const SwigluBwdArgs& a, hipStream_t st) {
    if (a.R == 0) return hipSuccess;
    const bool paired = ((a.I >> 3) % 64) == 32;
    const dim3 grid(grid_waves(paired ? (a.R + 1) / 2 : a.R));
#define FQ_SWIGLU_BWD(KIND)                                                                         \
    if (paired) hipLaunchKernelGGL((k_swiglu_bwd<KIND, 2>), grid, dim3(TPB), 0, st, a);             \
    else hipLaunchKernelGGL((k_swiglu_bwd<KIND, 1>), grid, dim3(TPB), 0, st, a);
    switch (a.a2.q.kind) {
    case K_NONE: FQ_SWIGLU_BWD(K_NONE); break;
    case K_NVFP4: FQ_SWIGLU_BWD(K_NVFP4); break;
    case K_INT: FQ_SWIGLU_BWD(K_INT); break;
    default: FQ_SWIGLU_BWD(K_FP8); break;
    }
#undef FQ_SWIGLU_BWD
    return hipGetLastError();
}

// waves per token in the A1 backward: a quarter row each when the row is a
// multiple of 256 vectors (H = 2048: one vector per lane), else a half row
// when a multiple of 128; each wave's ds_a1 partial is one of that many per row
int unpermute_split(int H) {
    const int nvec = H >> 3;
    if (nvec % 256 == 0) return 4;
    return (nvec % 128 == 0 && nvec >= 256) ? 2 : 1;
}

hipError_t launch_unpermute_a1(const UnpermuteArgs& a, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    const int split = unpermute_split(a.H);
    const dim3 grid(grid_waves(a.T * split));
    const int nv = nv_for(a.H / split);
    const int nv4 = a.H / split <= 512 ? 1 : nv;
#define FQ_UNPERM(KIND)                                                                                 \
    if (split == 4) {                                                                                   \
        switch (nv4) {                                                                                  \
        case 1: hipLaunchKernelGGL((k_unpermute_a1<KIND, 1, 4>), grid, dim3(TPB), 0, st, a); break;     \
        case 2: hipLaunchKernelGGL((k_unpermute_a1<KIND, 2, 4>), grid, dim3(TPB), 0, st, a); break;     \
        case 4: hipLaunchKernelGGL((k_unpermute_a1<KIND, 4, 4>), grid, dim3(TPB), 0, st, a); break;     \
        default: hipLaunchKernelGGL((k_unpermute_a1<KIND, 8, 4>), grid, dim3(TPB), 0, st, a); break;    \
        }                                                                                               \
    } else if (split == 2) {                                                                            \
        switch (nv) {                                                                                   \
        case 2: hipLaunchKernelGGL((k_unpermute_a1<KIND, 2, 2>), grid, dim3(TPB), 0, st, a); break;     \
        case 4: hipLaunchKernelGGL((k_unpermute_a1<KIND, 4, 2>), grid, dim3(TPB), 0, st, a); break;     \
        default: hipLaunchKernelGGL((k_unpermute_a1<KIND, 8, 2>), grid, dim3(TPB), 0, st, a); break;    \
        }                                                                                               \
    } else {                                                                                            \
        switch (nv) {                                                                                   \
        case 2: hipLaunchKernelGGL((k_unpermute_a1<KIND, 2, 1>), grid, dim3(TPB), 0, st, a); break;     \
        case 4: hipLaunchKernelGGL((k_unpermute_a1<KIND, 4, 1>), grid, dim3(TPB), 0, st, a); break;     \
        case 8: hipLaunchKernelGGL((k_unpermute_a1<KIND, 8, 1>), grid, dim3(TPB), 0, st, a); break;     \
        default: hipLaunchKernelGGL((k_unpermute_a1<KIND, 16, 1>), grid, dim3(TPB), 0, st, a); break;  \
        }                                                                                               \
    }
    switch (a.a1.q.kind) {
    case K_NONE: FQ_UNPERM(K_NONE); break;
    case K_NVFP4: FQ_UNPERM(K_NVFP4); break;
    case K_INT: FQ_UNPERM(K_INT); break;
    default: FQ_UNPERM(K_FP8); break;
    }
#undef FQ_UNPERM
    return hipGetLastError();
}

hipError_t launch_segment_sum(const float* rowpart, const int32_t* offsets, int E, int per, float* out,
                              hipStream_t st) {
    hipLaunchKernelGGL(k_segment_sum, dim3((unsigned)E), dim3(SEG_TPB), 0, st, rowpart, offsets, per, out);
    return hipGetLastError();
}

}  // namespace fq
