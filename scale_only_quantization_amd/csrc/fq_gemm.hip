// bf16 grouped GEMM over all experts on the gfx950 matrix cores (the single
// grouped GEMM of the nxmr.cn article on MCoreQAD, section 二.4).
//
// Three operand layouts share one kernel body:
//   FWD    C[r, n]    = sum_k A[r, k] B_e[n, k]      A routed rows, B [N, K]   (bf16 out)
//   DGRAD  C[r, n]    = sum_k A[r, k] B_e[k, n]      B stored [K, N]           (bf16 out)
//   WGRAD  C_e[i, j]  = sum_r A[r, i] B[r, j]        rows r of expert e        (fp32 out)
//
// Block: WVM x WVN waves; each wave owns WTM x WTN 32 x 32 output tiles
// (v_mfma_f32_32x32x16_bf16).  Large tile: 256 x 256 on 8 waves (2 x 4, each
// 128 x 64, two waves per SIMD); small tile: 128 x 128 on 4 waves.
//
// Operands go from global memory straight into LDS (buffer_load ... lds,
// 16 B per lane; one wave instruction fills 1 KB), through buffer resources
// bounded to the valid rows, so rows past the routed rows or past an expert's
// rows (the WGRAD reduction tail) read as zero.  A reduction step is BK deep;
// S LDS stages are in flight, so a tile's loads are issued S-1 steps before
// its MFMAs.  The stages of A come first in LDS, then those of B.  The large
// tiles run a ping-pong schedule (two groups of four waves, one phase apart;
// see mainloop_pp): FWD and DGRAD with BK = 64 and two stages, WGRAD with
// BK = 32 and three.
//   K-contiguous operand: LDS [rows][BK], the 16-B chunk index XORed with a
//     row swizzle; a fragment (8 consecutive k of one row) is one
//     ds_read_b128, and the 16 rows of one read pass fall on distinct banks.
//   Row-contiguous operand: LDS [BK][rows] as in memory, 16-B chunk c of k-row
//     k stored at chunk c ^ 2 (k & 3) ^ 8 (bit 1 of c); a fragment is two
//     ds_read_b64_tr_b16: inside each group of 16 lanes, lane i points at
//     k-row kb + i/4, columns mb + 4(i%4) .. +3, and lane j receives
//     k = kb .. kb+3 of column mb + j.  The swizzle spreads a group's 4 rows
//     over 8 chunks and puts the two groups of one 32-column half on opposite
//     halves of the banks: these reads then run at 140 B/clk per CU, against
//     107 with chunk c ^ 4 (k & 3) and 58 unswizzled (measured on gfx950).
// FWD/DGRAD row tiles come from a device-side tile table (expert, first row)
// built by the routing scan, so no host read-back of the counts is needed.
// WGRAD is persistent: each XCD works through its own experts' tiles (an
// assignment the routing scan balances), taken from a per-XCD counter.
#include <type_traits>

#include "fq_common.h"
#include "fq_internal.h"

#ifndef GEMM_BK_BIG
#define GEMM_BK_BIG 64      // reduction step and LDS stages of the large FWD/DGRAD tile
#define GEMM_S_BIG 2
#endif
#ifndef GEMM_BK_WG
#define GEMM_BK_WG 32       // the same for the large WGRAD tile
#define GEMM_S_WG 3
#endif
#ifndef GEMM_XCD
#define GEMM_XCD 1          // contiguous tile runs per XCD for FWD/DGRAD
#endif
#ifndef GEMM_WVM
#define GEMM_WVM 2          // waves of the large tile along rows x columns
#define GEMM_WVN 4
#endif
#ifndef GEMM_PP
#define GEMM_PP 1           // ping-pong schedule of the 8-wave tile (FWD, DGRAD)
#endif
#ifndef GEMM_PP_WG
#define GEMM_PP_WG 1        // the same for WGRAD
#endif

namespace fq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;


enum Mode { FWD = 0, DGRAD = 1, WGRAD = 2 };

// Buffer resource over [base, base + bytes): loads outside read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0xFFFFFFF0ll) bytes = 0xFFFFFFF0ll;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes,
                                             0x00020000);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The same resource as four wave-uniform dwords, for stage_load below.
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, int64_t bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0xFFFFFFF0ll) bytes = 0xFFFFFFF0ll;
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);     // stride 0
    r.z = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
    r.w = 0x00020000u;
    return r;
}

// One wave's direct global->LDS loads of a stage: N loads of 16 B per lane,
// load i from resource offset voff[i] + soff into the 1 KB of LDS at
// dst + i * STEP (dst wave-uniform; lane l writes 16 B at + 16 l).  Written as
// assembly so that the compiler does not see LDS writes in flight: it would
// otherwise wait for every such load (vmcnt(0)) before the next transposing
// LDS read, i.e. put the latency of the step's loads just issued in front of
// the current step's fragment reads.  Callers order these loads against the
// LDS reads themselves, with their own vmcnt waits and barriers.  M0 carries
// each load's LDS address (one wait state between its write and the load);
// the leading s_nop 4 gives the five wait states a vector-memory read of an
// SGPR needs after a vector instruction wrote it (v_readfirstlane, or
// v_readlane restoring a spilled SGPR), which the compiler supplies for its
// own instructions but not for assembly.
template <int N, int STEP>
__device__ __forceinline__ void stage_loads(const u32x4& rs, lds_t* dst, const uint32_t (&voff)[N], uint32_t soff) {
    static_assert(N >= 1 && N <= 4, "loads per wave and stage");
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
#define FQ_LDS_LOAD(V) "s_nop 0\n\tbuffer_load_dwordx4 " V ", %[r], %[so] offen lds\n\t"
    if constexpr (N == 1) {
        asm volatile("s_nop 4\n\ts_mov_b32 m0, %[m]\n\t" FQ_LDS_LOAD("%[v0]")
                     :
                     : [m] "s"(m), [v0] "v"(voff[0]), [r] "s"(rs), [so] "s"(soff)
                     : "memory", "m0");
    } else if constexpr (N == 2) {
        asm volatile("s_nop 4\n\ts_mov_b32 m0, %[m]\n\t" FQ_LDS_LOAD("%[v0]")
                     "s_add_i32 m0, %[m], %[d1]\n\t" FQ_LDS_LOAD("%[v1]")
                     :
                     : [m] "s"(m), [v0] "v"(voff[0]), [v1] "v"(voff[1]), [r] "s"(rs), [so] "s"(soff),
                       [d1] "n"(STEP)
                     : "memory", "m0");
    } else if constexpr (N == 3) {
        asm volatile("s_nop 4\n\ts_mov_b32 m0, %[m]\n\t" FQ_LDS_LOAD("%[v0]")
                     "s_add_i32 m0, %[m], %[d1]\n\t" FQ_LDS_LOAD("%[v1]")
                     "s_add_i32 m0, %[m], %[d2]\n\t" FQ_LDS_LOAD("%[v2]")
                     :
                     : [m] "s"(m), [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [r] "s"(rs),
                       [so] "s"(soff), [d1] "n"(STEP), [d2] "n"(2 * STEP)
                     : "memory", "m0");
    } else {
        asm volatile("s_nop 4\n\ts_mov_b32 m0, %[m]\n\t" FQ_LDS_LOAD("%[v0]")
                     "s_add_i32 m0, %[m], %[d1]\n\t" FQ_LDS_LOAD("%[v1]")
                     "s_add_i32 m0, %[m], %[d2]\n\t" FQ_LDS_LOAD("%[v2]")
                     "s_add_i32 m0, %[m], %[d3]\n\t" FQ_LDS_LOAD("%[v3]")
                     :
                     : [m] "s"(m), [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]),
                       [r] "s"(rs), [so] "s"(soff), [d1] "n"(STEP), [d2] "n"(2 * STEP), [d3] "n"(3 * STEP)
                     : "memory", "m0");
    }
#undef FQ_LDS_LOAD
}

// x of lane l ^ 32: one cross-half swap (v_permlane32_swap) and a select, no
// LDS round trip.  The swap returns (lanes 0-31 of x in both halves, lanes
// 32-63 of x in both halves).
__device__ __forceinline__ float xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Wait until at most n (clamped to 0..3) steps of L load instructions each
// are outstanding: vector-memory loads complete in issue order.
template <int L>
__device__ __forceinline__ void wait_steps(int n) {
    static_assert(3 * L <= 63, "vmcnt range");
    if (n <= 0) vm_wait<0>();
    else if (n == 1) vm_wait<L>();
    else if (n == 2) vm_wait<2 * L>();
    else vm_wait<3 * L>();
}

// K-contiguous operand tile [ROWS][BK]: element (row, k) at byte row*ld2 + 2k
// of the resource.  Rows of 2 BK bytes; each 1-KB wave load covers 512/BK rows.
// Swizzle: chunk ^ (row >> 2) & 3 for 64-B rows, chunk ^ (row >> 1) & 7 for
// 128-B rows, so the 16 rows one ds_read_b128 pass serves (16 lanes x 16 B,
// 64 banks) fall on distinct banks; rows 32 apart share a swizzle, so a
// wave's fragments of one k sub-step differ by constant offsets.
template <int ROWS, int BK, int NW>
struct KTile {
    static constexpr int BYTES = ROWS * BK * 2;
    static constexpr int PER_WAVE = BYTES / 1024 / NW;
    static constexpr int CPR = BK / 8;                 // 16-B chunks per row
    static constexpr int RB = 2 * BK;                  // bytes per row
    static constexpr int KS = BK / 16;                 // 16-deep sub-steps per step
    __device__ static __forceinline__ int swz(int row) {
        return BK == 32 ? ((row >> 2) & 3) : ((row >> 1) & 7);
    }
    __device__ static __forceinline__ int off(int row, int ch) {   // byte offset of 16-B chunk
        return row * RB + ((ch ^ swz(row)) << 4);
    }
    u32x4 rs;
    uint32_t voff[PER_WAVE];
    __device__ __forceinline__ void init(const u32x4& r, int64_t ld) {
        rs = r;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int blk = NW * i + w;                   // 1-KB block
            const int row = blk * (64 / CPR) + lane / CPR;
            const int lc = (lane % CPR) ^ swz(row);       // logical chunk stored at this position
            voff[i] = (uint32_t)(row * ld * 2 + lc * 16);
        }
    }
    __device__ __forceinline__ void issue(lds_t* tile, int k0) {
        stage_loads<PER_WAVE, NW * 1024>(rs, tile + wave_id() * 1024, voff, (uint32_t)k0 * 2);
    }
    // fragment of the 32x32x16 MFMA: row `row0 + lane%32`, k = 16 kk + 8 (lane/32) .. +7
    __device__ static __forceinline__ bf16x8 frag(const lds_t* tile, int row0, int kk) {
        const int lane = threadIdx.x & 63;
        const int row = row0 + (lane & 31);
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            tile + off(row, kk * 2 + (lane >> 5)));
    }
    // A wave's fragments from per-lane offsets: one offset per sub-step kk for
    // rows row0w + 32 t + lane%32 (row0w a multiple of 32); t adds 32 RB.
    template <int WT>
    struct Frags {
        uint32_t o[KS];
        __device__ __forceinline__ void prep(int row0w) {
            const int lane = threadIdx.x & 63;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) o[kk] = (uint32_t)off(row0w + (lane & 31), kk * 2 + (lane >> 5));
        }
        __device__ __forceinline__ bf16x8 get(const lds_t* tile, int t, int kk) const {
            return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + o[kk] + t * 32 * RB);
        }
    };
};

// Row-contiguous operand tile [BK][ROWS] (stored as in memory): element
// (row, k) at byte k*ld2 + 2*row of the resource.  Each 1-KB wave load covers
// 1024 / (2 ROWS) k-rows.
template <int ROWS, int BK, int NW>
struct MNTile {
    static constexpr int BYTES = ROWS * BK * 2;
    static constexpr int PER_WAVE = BYTES / 1024 / NW;
    static constexpr int RB = ROWS * 2;               // bytes per k-row
    // 16-B chunk ch of k-row k is stored at chunk ch ^ 2 (k & 3) ^ 8 (bit 1 of ch)
    __device__ static __forceinline__ int phys(int k, int ch) { return ch ^ ((k & 3) << 1) ^ (((ch >> 1) & 1) << 3); }
    __device__ static __forceinline__ int off(int k, int byte) {   // swizzled byte offset
        return k * RB + (phys(k, byte >> 4) << 4) + (byte & 15);
    }
    u32x4 rs;
    uint32_t voff[PER_WAVE];
    uint32_t ld2;
    __device__ __forceinline__ void init(const u32x4& r, int64_t ld) {
        rs = r;
        ld2 = (uint32_t)(ld * 2);
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int pos = (NW * i + w) * 1024 + lane * 16;  // byte position in the tile
            const int k = pos / RB;
            const int pc = (pos % RB) >> 4;
            const int lc = pc ^ ((k & 3) << 1) ^ ((((pc >> 1) ^ k) & 1) << 3);   // phys(k, lc) == pc
            voff[i] = (uint32_t)(k * ld * 2 + lc * 16);
        }
    }
    __device__ __forceinline__ void issue(lds_t* tile, int k0) {
        stage_loads<PER_WAVE, NW * 1024>(rs, tile + wave_id() * 1024, voff, (uint32_t)k0 * ld2);
    }
    __device__ static __forceinline__ bf16x8 frag(const lds_t* tile, int row0, int kk) {
        const int lane = threadIdx.x & 63;
        const int i = lane & 15;
        const int mb = row0 + ((lane >> 4) & 1) * 16;
        const int kb = kk * 16 + (lane >> 5) * 8 + (i >> 2);
        const int byte = (mb + 4 * (i & 3)) * 2;
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
        typedef __attribute__((address_space(3))) v4bf lds4;
        lds_t* t = const_cast<lds_t*>(tile);
        const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(t + off(kb, byte))));
        const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(t + off(kb + 4, byte))));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // A wave's fragments from per-lane offsets: one offset per 32-row tile t
    // (rows row0w + 32 t); sub-step kk adds 16 k-rows, the second read 4.
    template <int WT>
    struct Frags {
        uint32_t o[WT];
        __device__ __forceinline__ void prep(int row0w) {
            const int lane = threadIdx.x & 63;
            const int i = lane & 15;
            const int kb = (lane >> 5) * 8 + (i >> 2);
#pragma unroll
            for (int t = 0; t < WT; ++t) {
                const int mb = row0w + 32 * t + ((lane >> 4) & 1) * 16;
                o[t] = (uint32_t)off(kb, (mb + 4 * (i & 3)) * 2);
            }
        }
        __device__ __forceinline__ bf16x8 get(const lds_t* tile, int t, int kk) const {
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
            typedef __attribute__((address_space(3))) v4bf lds4;
            lds_t* p = const_cast<lds_t*>(tile) + o[t] + kk * 16 * RB;
            const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)p));
            const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(p + 4 * RB)));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
};

// Block -> tile with XCD locality: workgroups are dealt to the 8 XCDs (each
// with its own L2) round-robin, so XCD x = id % 8 is given the contiguous run
// of tiles [x * chunk, (x + 1) * chunk), chunk = ceil(tiles / 8); tiles that
// share operands (the N tiles of one row tile, the row tiles of one expert)
// then meet in the same L2.  Returns -1 for ids past the tile count.
__device__ __forceinline__ int xcd_tile(int id, int grid, int tiles) {
    const int chunk = (tiles + 7) / 8;
    const int t = (id % 8) * chunk + id / 8;
    return (id / 8 < chunk && t < tiles) ? t : -1;
}

// sum of g c over 8 elements sharing the effective scale s.  On the fast
// path (every lane's scale normal) the NVFP4 grid value is converted from the
// signed quotient directly (the conversion saturates): c = q - r only needs
// q's value, and a zero element has c = 0 whatever the sign of its q.
template <int KIND>
__device__ __forceinline__ float sg_part8(const float* w8, const float* g8, float s, float qmin, float qmax) {
    float part = 0.0f;
    if (KIND == K_NVFP4) {
        // every lane's scale normal: the corrected reciprocal quotient (the
        // IEEE division of the general path is not evaluated)
        if (__all(s >= 0x1p-120f && s <= 0x1p120f)) {
            const float inv = rcp_rn(s);
            float r[8], q[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float q0 = w8[v] * inv;
                r[v] = __builtin_fmaf(__builtin_fmaf(-q0, s, w8[v]), inv, q0);
            }
            e2m1_round8(r, q);
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float c = q[v] - (fabsf(r[v]) <= 6.0f ? r[v] : 0.0f);
                part = __builtin_fmaf(g8[v], c, part);
            }
            return part;
        }
    }
    quant_group<KIND, 8>(w8, s, qmin, qmax, [&](int v, const Elem& el) {
        part = __builtin_fmaf(g8[v], ste_c(el, qmin, qmax), part);
    });
    return part;
}

// fl32(s / t) for the NVFP4 block factor: Markstein's corrected quotient from
// inv_t = RN(1/t) when t is normal (the caller's wave-uniform tfast), IEEE
// division otherwise
__device__ __forceinline__ float div_by_t(float s, float t, float inv_t, bool tfast) {
    if (tfast) {
        const float q0 = s * inv_t;
        return __builtin_fmaf(__builtin_fmaf(-q0, t, s), inv_t, q0);
    }
    return s / t;
}

// Weight-gradient epilogue with the weight-scale gradient fused: the wave's
// accumulators are dW_e[i, j] for rows i = i_w + 32 ti + lane%32 and columns
// j = j_w + 32 tj + 8 q + 4 (lane/32) + v.  Each element's straight-through
// term c is recomputed from the frozen weight and its effective scale exactly
// as the fake-quant backward does, and g c is summed per 16-column block
// (a block is q = 2b, 2b+1 of both lane halves) or per 32-column tile.
template <int KIND, int WTM, int WTN>
__device__ __forceinline__ void sg_epilogue(const GemmArgs& g, const f32x16 (&acc)[WTM][WTN], int e,
                                            int i_w, int j_w, int lane) {
    const SgArgs& sg = g.sg;
    const int64_t N = g.N, K = g.K;
    const float qmin = sg.q.qmin, qmax = sg.q.qmax;
    const int gran = sg.q.gran, group = sg.q.group;
    const float t = KIND == K_NVFP4 ? sg.tscale[e] : 0.0f;
    // weights and scales of 32-row slice ti are fetched while slice ti-1 is
    // reduced: one memory round trip per slice instead of one per element group
    uint2 wv[2][WTN][4];
    float sv[2][WTN][2];
    auto fetch = [&](int ti, int buf) {
        const int64_t wrow = (int64_t)e * N + i_w + ti * 32 + (lane & 31);
        const uint16_t* Wr = sg.W + wrow * K;
#pragma unroll
        for (int tj = 0; tj < WTN; ++tj) {
            const int jt = j_w + tj * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                wv[buf][tj][q] = *reinterpret_cast<const uint2*>(Wr + jt + 8 * q + 4 * (lane >> 5));
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int j = jt + 16 * b;
                if (KIND == K_NVFP4) sv[buf][tj][b] = sg.scale[wrow * (K >> 4) + (j >> 4)];
                else if (gran == G_GROUP) sv[buf][tj][b] = sg.scale[wrow * (K / group) + j / group];
                else if (gran == G_ROW) sv[buf][tj][b] = sg.scale[wrow];
                else sv[buf][tj][b] = sg.scale[e];
            }
        }
    };
    fetch(0, 0);
#pragma unroll
    for (int ti = 0; ti < WTM; ++ti) {
        const int cur = ti & 1;
        if (ti + 1 < WTM) fetch(ti + 1, cur ^ 1);
        const int64_t wrow = (int64_t)e * N + i_w + ti * 32 + (lane & 31);
#pragma unroll
        for (int tj = 0; tj < WTN; ++tj) {
            const int jt = j_w + tj * 32;
            float p[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                // effective scale of the 16-column block (the block's columns
                // share one scale for every granularity allowed here)
                float s = sv[cur][tj][b];
                if (KIND == K_NVFP4) s = t * e4m3_round(fminf(s / t, 448.0f));
                // this lane's 8 elements of the block: q = 2b, 2b+1, 4 columns each
                const uint2 wa = wv[cur][tj][2 * b], wb = wv[cur][tj][2 * b + 1];
                const float w8[8] = {bf_lo(wa.x), bf_hi(wa.x), bf_lo(wa.y), bf_hi(wa.y),
                                     bf_lo(wb.x), bf_hi(wb.x), bf_lo(wb.y), bf_hi(wb.y)};
                float g8[8];
#pragma unroll
                for (int v = 0; v < 8; ++v) g8[v] = acc[ti][tj][8 * b + v];
                p[b] = sg_part8<KIND>(w8, g8, s, qmin, qmax);
            }
            const float b0 = p[0] + xor32(p[0]);
            const float b1 = p[1] + xor32(p[1]);
            if (lane < 32) {
                if (!sg.part32) {
                    float* o = sg.out + wrow * (K >> 4) + (jt >> 4);   // 4-byte aligned only
                    o[0] = b0;
                    o[1] = b1;
                } else {
                    sg.out[wrow * (K >> 5) + (jt >> 5)] = b0 + b1;
                }
            }
        }
    }
}

// Frozen weights of the fused epilogue staged through LDS: each wave owns two
// 4-KB slots, each one 32-row slice of its 64 columns (bf16), filled by direct
// global->LDS loads so that no registers wait on them.  16-B chunks of a row
// are XOR-swizzled by (row >> 1) & 7: the 64 lanes' 8-B reads of one column
// group then cover all 64 banks twice, the minimum for 512 B.
struct WStage {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t K2;                                       // bytes per weight row
    // w0: element (row 0, column 0) of the wave's block; rows x 64 columns
    __device__ __forceinline__ void init(const uint16_t* w0, int64_t K, int rows) {
        rs = make_rsrc(w0, ((int64_t)(rows - 1) * K + 64) * 2);
        K2 = (uint32_t)(K * 2);
    }
    // rows 32 ti .. 32 ti + 31 into `slot`: 4 wave loads of 1 KB
    __device__ __forceinline__ void issue(lds_t* slot, int ti) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = i * 64 + lane;
            const int r = p >> 3;
            const int c = (p & 7) ^ ((r >> 1) & 7);            // logical chunk at this position
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, slot + i * 1024, 16,
                                                     (uint32_t)(ti * 32 + r) * K2 + (uint32_t)c * 16, 0, 0, 0);
        }
    }
    // this lane's 4 weights of chunk c (columns 8 c + 4 (lane / 32) .. +3, row lane % 32)
    __device__ static __forceinline__ uint2 read(const lds_t* slot, int c) {
        const int lane = threadIdx.x & 63;
        const int r = lane & 31;
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
            slot + r * 128 + ((c ^ ((r >> 1) & 7)) << 4) + (lane >> 5) * 8);
        return make_uint2(v.x, v.y);
    }
};

// The epilogue above with the weights read from the wave's LDS slots, in two
// parts.  begin(): the scales of slices 0 and 1 (issued after slices 0 and 1
// of the weights).  run(): waits until at most `later` steps of L loads are
// outstanding, calls after_wait() (which issues the next tile's first loads),
// then reduces slice by slice; slice ti + 2 refills slice ti's slot as soon
// as slice ti's weights are in registers.  A wait on the vector memory
// counter also covers the direct-to-LDS loads; this wave alone reads its
// slots.
template <int KIND, int WTM, int WTN>
struct SgEpiLds {
    static_assert(WTN == 2 && WTM >= 2, "two 32-column tiles per wave, two slots");
    float sv[WTM][WTN][2];
    // scales of slice ti (the loads' waits are the compiler's): the row's four
    // 16-column blocks are one 16-B load when each block has its own scale
    __device__ __forceinline__ void load_sv(const GemmArgs& g, int e, int i_w, int j_w, int lane, int ti) {
        const SgArgs& sg = g.sg;
        const int64_t N = g.N, K = g.K;
        const int gran = sg.q.gran, group = sg.q.group;
        const int64_t wrow = (int64_t)e * N + i_w + ti * 32 + (lane & 31);
        if (KIND == K_NVFP4 || (gran == G_GROUP && group == 16)) {
            typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
            const f32x4u v = *reinterpret_cast<const f32x4u*>(sg.scale + wrow * (K >> 4) + (j_w >> 4));
            sv[ti][0][0] = v.x;
            sv[ti][0][1] = v.y;
            sv[ti][1][0] = v.z;
            sv[ti][1][1] = v.w;
            return;
        }
        if (gran != G_GROUP) {
            // one scale for the slice's row (or the matrix), read where used
            // (copying it here would wait for the load at once)
            sv[ti][0][0] = sg.scale[gran == G_ROW ? wrow : (int64_t)e];
            return;
        }
#pragma unroll
        for (int tj = 0; tj < WTN; ++tj)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int j = j_w + tj * 32 + 16 * b;
                sv[ti][tj][b] = sg.scale[wrow * (K / group) + j / group];
            }
    }
    __device__ __forceinline__ void begin(const GemmArgs& g, int e, int i_w, int j_w, int lane) {
        load_sv(g, e, i_w, j_w, lane, 0);
        load_sv(g, e, i_w, j_w, lane, 1);
    }
    // after_wait(): called once the first two slices and scales have landed
    // (loads it issues overlap the reductions)
    template <int L, typename F>
    __device__ __forceinline__ void run(const GemmArgs& g, const f32x16 (&acc)[WTM][WTN], int e, int i_w, int j_w,
                                        int lane, const WStage& ws, lds_t* slots, int later, F&& after_wait) {
        const SgArgs& sg = g.sg;
        const int64_t N = g.N, K = g.K;
        const float qmin = sg.q.qmin, qmax = sg.q.qmax;
        // t is one per expert: read into a scalar register, so that the
        // branch on its range below is a wave-uniform jump
        const float t = KIND == K_NVFP4 ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sg.tscale[e])))
                                        : 0.0f;
        const bool tfast = t >= 0x1p-120f && t <= 0x1p120f;
        const float inv_t = KIND == K_NVFP4 ? rcp_rn(t) : 0.0f;
        wait_steps<L>(later);
        after_wait();
#pragma unroll
        for (int ti = 0; ti < WTM; ++ti) {
            lds_t* slot = slots + (ti & 1) * 4096;
            if (ti == 2) vm_wait<0>();                  // slices 2 and 3 have landed
            const int64_t wrow = (int64_t)e * N + i_w + ti * 32 + (lane & 31);
            uint2 wv[WTN][4];
#pragma unroll
            for (int tj = 0; tj < WTN; ++tj)
#pragma unroll
                for (int q = 0; q < 4; ++q) wv[tj][q] = WStage::read(slot, 4 * tj + q);
            if (ti + 2 < WTM) {
                load_sv(g, e, i_w, j_w, lane, ti + 2);
                // the slot's reads have returned before it is refilled
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                ws.issue(slot, ti + 2);
            }
#pragma unroll
            for (int tj = 0; tj < WTN; ++tj) {
                const int jt = j_w + tj * 32;
                float p[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    float sc = sg.q.gran != G_GROUP ? sv[ti][0][0] : sv[ti][tj][b];
                    if (KIND == K_NVFP4) sc = t * e4m3_round(fminf(div_by_t(sc, t, inv_t, tfast), 448.0f));
                    const uint2 wa = wv[tj][2 * b], wb = wv[tj][2 * b + 1];
                    const float w8[8] = {bf_lo(wa.x), bf_hi(wa.x), bf_lo(wa.y), bf_hi(wa.y),
                                         bf_lo(wb.x), bf_hi(wb.x), bf_lo(wb.y), bf_hi(wb.y)};
                    float g8[8];
#pragma unroll
                    for (int v = 0; v < 8; ++v) g8[v] = acc[ti][tj][8 * b + v];
                    p[b] = sg_part8<KIND>(w8, g8, sc, qmin, qmax);
                }
                const float b0 = p[0] + xor32(p[0]);
                const float b1 = p[1] + xor32(p[1]);
                if (lane < 32) {
                    if (!sg.part32) {
                        float* o = sg.out + wrow * (K >> 4) + (jt >> 4);
                        o[0] = b0;
                        o[1] = b1;
                    } else {
                        sg.out[wrow * (K >> 5) + (jt >> 5)] = b0 + b1;
                    }
                }
            }
        }
    }
};

template <int MODE, int WVM, int WVN, int WTM, int WTN, int BK, int S>
__global__ __launch_bounds__(64 * WVM * WVN) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(GemmArgs g) {
    constexpr int NW = WVM * WVN;
    constexpr int BM = 32 * WTM * WVM, BN = 32 * WTN * WVN;
    typedef typename std::conditional<MODE == WGRAD, MNTile<BM, BK, NW>, KTile<BM, BK, NW>>::type ATile;
    typedef typename std::conditional<MODE == FWD, KTile<BN, BK, NW>, MNTile<BN, BK, NW>>::type BTile;
    constexpr int A_BYTES = ATile::BYTES, B_BYTES = BTile::BYTES;
    constexpr int LOADS = ATile::PER_WAVE + BTile::PER_WAVE;     // wave load instructions per stage
    constexpr int KS = BK / 16;                                  // 16-deep sub-steps per step
    static_assert(S >= 2 && S <= 4, "stages");
    // LDS: the S stages of A, then the S stages of B (a stage's offset then
    // fits a read's immediate); FWD/DGRAD reuse it for the bf16 output tile
    constexpr int STAGES = S * (A_BYTES + B_BYTES);
    constexpr int SMEM = (MODE != WGRAD && BM * BN * 2 > STAGES) ? BM * BN * 2 : STAGES;
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
    lds_t* smem = (lds_t*)smem_raw;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WVN, wn = wave % WVN;

    ATile la;
    BTile lb;
    // this wave's fragment offsets inside a stage (formed at the start of each
    // main loop, so they are not live across the weight-gradient epilogue)
    typename ATile::template Frags<WTM> fa;
    typename BTile::template Frags<WTN> fb;
    f32x16 acc[WTM][WTN];
    auto zero_acc = [&]() {
#pragma unroll
        for (int a = 0; a < WTM; ++a)
#pragma unroll
            for (int b = 0; b < WTN; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    };
    auto stage_a = [&](int kt) { return smem + (kt % S) * A_BYTES; };
    auto stage_b = [&](int kt) { return smem + S * A_BYTES + (kt % S) * B_BYTES; };

    // MFMAs of one BK-deep step: fragments of the next 16-deep sub-step are
    // read while the current sub-step's MFMAs run.
    auto compute = [&](int kt) {
        const lds_t* sa = stage_a(kt);
        const lds_t* sb = stage_b(kt);
        bf16x8 af[2][WTM], bfr[2][WTN];
#pragma unroll
        for (int kk = 0; kk <= KS; ++kk) {
            if (kk < KS) {
#pragma unroll
                for (int t = 0; t < WTM; ++t) af[kk & 1][t] = fa.get(sa, t, kk);
#pragma unroll
                for (int t = 0; t < WTN; ++t) bfr[kk & 1][t] = fb.get(sb, t, kk);
            }
            if (kk > 0) {
                const int s = (kk - 1) & 1;
#pragma unroll
                for (int ti = 0; ti < WTM; ++ti)
#pragma unroll
                    for (int tj = 0; tj < WTN; ++tj)
                        acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s][tj], af[s][ti], acc[ti][tj],
                                                                              0, 0, 0);
            }
        }
        constexpr int NR = WTM * (std::is_same<ATile, KTile<BM, BK, NW>>::value ? 1 : 2) +
                           WTN * (std::is_same<BTile, KTile<BN, BK, NW>>::value ? 1 : 2);
        constexpr int NM = WTM * WTN;
        // each sub-step: the next sub-step's reads first, then its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    };
    auto issue = [&](int kt) {
        la.issue(stage_a(kt), kt * BK);
        lb.issue(stage_b(kt), kt * BK);
    };
    // steps [p0, p1] of this wave's loads (those below nk)
    auto issue_steps = [&](int nk, int p0, int p1) {
#pragma unroll
        for (int p = 0; p < S; ++p)
            if (p >= p0 && p <= p1 && p < nk) issue(p);
    };
    // Single-phase loop: every wave waits for step kt, one barrier, then the
    // loads of step kt+S-1 and the MFMAs of step kt.  pre: steps [0, pre)
    // were issued before the call (into stages the caller may have used
    // since, hence the barrier before the rest of the prologue).
    // first(): called once, after the first step's loads are issued (memory
    // operations it starts overlap the first step)
    auto mainloop = [&](int nk, int pre, auto&& first) {
        fa.prep(wm * 32 * WTM);
        fb.prep(wn * 32 * WTN);
        if (pre > 0) __syncthreads();
        issue_steps(nk, pre, S - 2);
        if (nk <= 0) first();
        for (int kt = 0; kt < nk; ++kt) {
            // this wave's loads of step kt are done once at most those of the
            // later steps already issued are outstanding; the barrier then
            // covers every wave
            wait_steps<LOADS>(min(S - 2, nk - 1 - kt));
            __syncthreads();
            // the stage step kt+S-1 overwrites was read in step kt-1, finished by every wave
            if (kt + S - 1 < nk) issue(kt + S - 1);
            if (kt == 0) first();
            compute(kt);
        }
    };

    // Ping-pong schedule of the 8-wave tile.  Waves 0-3 (group 0) and 4-7
    // (group 1), one of each per SIMD, alternate between a memory phase
    // (every fragment of one BK step read from LDS into registers, and this
    // wave's global loads) and a compute phase (that step's MFMAs from
    // registers), group 1 one phase behind.  Between two barriers one wave on
    // each SIMD issues MFMAs while the other reads LDS and waits on memory, so
    // the matrix core does not idle across the barrier and the fragment reads
    // that follow it.
    //   group 0, memory phase of step kt: its loads of step kt+S-1 (into the
    //     stage step kt-1 used, read by both groups in the two phases
    //     before), then its fragment reads of step kt; it waits for its loads
    //     of step kt+1 after its next compute phase.
    //   group 1, memory phase of step kt: its fragment reads of step kt, then
    //     (once they have returned) its loads of step kt+S into the same stage
    //     (group 0 read it one phase earlier), then it waits for its loads of
    //     step kt+1.
    // Every load of step kt+1 has landed before the barrier that opens group
    // 0's memory phase of step kt+1.  Prologue: group 0 has steps [0, S-2] in
    // flight, group 1 steps [0, S-1]; pre: steps [0, pre) were issued by every
    // wave before the call.
    // The weight gradient runs it with 32-deep steps and three stages: with
    // 64-deep steps a step's fragments (both operands read transposed) do not
    // fit the registers beside the accumulators, and with three 32-deep
    // stages its loads have the same lead in time as two 64-deep ones.
    constexpr bool PP = GEMM_PP && NW == 8 && WVM == 2 && (MODE != WGRAD || GEMM_PP_WG);
    // nti: this wave's 32-row sub-tiles that hold valid rows (wave-uniform);
    // below WTM the MFMAs and fragment reads of the others are skipped
    auto mainloop_pp = [&](int nk, int pre, int nti, auto&& first, auto&& tail0) {
        const int grp = wave_id() >> 2;
        bf16x8 af[KS][WTM], bfr[KS][WTN];
        fa.prep(wm * 32 * WTM);
        fb.prep(wn * 32 * WTN);
        auto bar = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        if (pre > 0) bar();
        const int last = grp == 0 ? S - 2 : S - 1;
        issue_steps(nk, pre, last);
        wait_steps<LOADS>(min(last, nk - 1));
        bar();
        if (grp == 1) bar();
        auto phases = [&](int kt, int st, auto part_c) {
            constexpr bool PART = decltype(part_c)::value;
            // memory phase
            if (grp == 0 && kt + S - 1 < nk) issue(kt + S - 1);
            const lds_t* sa = smem + st * A_BYTES;
            const lds_t* sb = smem + S * A_BYTES + st * B_BYTES;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
                for (int t = 0; t < WTM; ++t)
                    if (!PART || t < nti) af[kk][t] = fa.get(sa, t, kk);
                if (!PART || nti > 0)
#pragma unroll
                    for (int t = 0; t < WTN; ++t) bfr[kk][t] = fb.get(sb, t, kk);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (grp == 1) {
                if (kt + S < nk) issue(kt + S);
                wait_steps<LOADS>(min(S - 1, nk - 2 - kt));
            }
            bar();
            // compute phase
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int ti = 0; ti < WTM; ++ti)
                    if (!PART || ti < nti)
#pragma unroll
                        for (int tj = 0; tj < WTN; ++tj)
                            acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk][tj], af[kk][ti],
                                                                                  acc[ti][tj], 0, 0, 0);
            if (grp == 0) wait_steps<LOADS>(min(S - 2, nk - 2 - kt));
            bar();
        };
        first();
        // full sub-tile sets keep the unpredicated loop
        auto steps = [&](auto part_c) {
            for (int kt = 0; kt < nk; kt += S) {
#pragma unroll
                for (int u = 0; u < S; ++u)
                    if (kt + u < nk) phases(kt + u, u, part_c);
            }
        };
        if (MODE == WGRAD || nti >= WTM) steps(std::false_type{});
        else steps(std::true_type{});
        // group 0 is done; while group 1 runs its last compute phase (no LDS
        // reads, no loads in flight) group 0 may use LDS
        if (grp == 0) {
            tail0();
            bar();
        }
    };
    auto no_hook = []() {};

    if constexpr (MODE != WGRAD) {
        const int ntn = g.N / BN;
        const int tile = GEMM_XCD ? xcd_tile(blockIdx.x, gridDim.x, g.num_tiles[0] * ntn) : (int)blockIdx.x;
        if (tile < 0 || tile >= g.num_tiles[0] * ntn) return;
        const int mt = tile / ntn;
        const int nt = tile - mt * ntn;
        const int e = min(max(g.tile_expert[mt], 0), g.E - 1);
        const int64_t m0 = g.tile_row0[mt];
        const int64_t m_end = min((int64_t)g.offsets[e + 1], g.R);   // the tile's expert's rows
        const int n0 = nt * BN;
        const int nk = g.K / BK;
        // rows past the expert's rows read as zero, without memory traffic
        // (their outputs are not stored)
        la.init(make_rsrc_words(g.A + m0 * g.lda, max(m_end - m0, (int64_t)0) * g.lda * 2), g.lda);
        const uint16_t* Be = g.B + (int64_t)e * g.strideB;
        if constexpr (MODE == FWD)
            lb.init(make_rsrc_words(Be + (int64_t)n0 * g.ldb, (int64_t)BN * g.ldb * 2), g.ldb);
        else
            lb.init(make_rsrc_words(Be + n0, ((int64_t)g.K - 1) * g.ldb * 2 + (int64_t)BN * 2), g.ldb);
        zero_acc();
        // Epilogue through LDS, so that global stores are whole row segments:
        // lane holds C[m = lane%32][n = 8*(v/4) + 4*(lane/32) + v%4] of each
        // 32x32 tile; it is written as bf16 into an LDS tile [BM][BN] whose
        // 16-B chunks are XOR-swizzled by (row & 15), then each wave copies
        // two rows per instruction (16 B per lane) to C.
        constexpr int RB = BN * 2, CH = BN / 8;                 // row bytes, 16-B chunks per row
        static_assert(BM * RB <= SMEM, "C tile fits the LDS");
        auto write_c = [&]() {
#pragma unroll
            for (int ti = 0; ti < WTM; ++ti) {
                const int row = wm * 32 * WTM + ti * 32 + (lane & 31);
#pragma unroll
                for (int tj = 0; tj < WTN; ++tj) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = wn * 32 * WTN + tj * 32 + 8 * q + 4 * (lane >> 5);
                        const int off = row * RB + (((col >> 3) ^ (row & 15)) << 4) + (col & 7) * 2;
                        *reinterpret_cast<__attribute__((address_space(3))) uint64_t*>(smem + off) =
                            (uint64_t)pack_bf16(acc[ti][tj][4 * q], acc[ti][tj][4 * q + 1]) |
                            ((uint64_t)pack_bf16(acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]) << 32);
                    }
                }
            }
        };
        if constexpr (PP) {
            // group 0 (rows 0..BM/2) writes its rows during group 1's last
            // compute phase, group 1 after it
            // rows of this wave's sub-tiles that hold routed rows of the expert
            const int wrows = (int)min((int64_t)BM, m_end - m0) - wm * 32 * WTM;
            mainloop_pp(nk, 0, min(max((wrows + 31) / 32, 0), WTM), no_hook, write_c);
            if (wave_id() >= 4) write_c();
        } else {
            mainloop(nk, 0, no_hook);
            __syncthreads();                                     // every wave is done with the stages
            write_c();
        }
        __syncthreads();
        constexpr int RPI = 64 / CH;                             // rows per wave instruction
        constexpr int NIT = BM / (RPI * NW);                     // store instructions per wave
        // every row segment of this wave from LDS first (one wait), then the
        // stores through a resource bounded to the tile's expert rows, so the
        // rows past m_end are dropped without branches; non-temporal (the
        // output is next read by another kernel)
        u32x4 cv[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int row = (it * NW + wave) * RPI + lane / CH;
            const int c = lane % CH;
            cv[it] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                smem + row * RB + ((c ^ (row & 15)) << 4));
        }
        const __amdgpu_buffer_rsrc_t crs =
            make_rsrc(static_cast<uint16_t*>(g.C) + m0 * g.ldc + n0, (m_end - m0 - 1) * g.ldc * 2 + BN * 2);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int row = (it * NW + wave) * RPI + lane / CH;
            const int c = lane % CH;
            __builtin_amdgcn_raw_buffer_store_b128(cv[it], crs, (uint32_t)(row * g.ldc * 2 + c * 16), 0, 2);
        }
    } else {
        // Persistent: the blocks of XCD group x = blockIdx % 8 (dealt to XCD x)
        // take the tiles of that XCD's experts (longest first) from a counter,
        // so the tiles sharing an expert's operand rows meet in one L2.  The
        // next tile's first loads are issued during this tile's epilogue (with
        // the fused scale gradient: once its first weights and scales have
        // landed; without it: before it).
        // Slots are taken one tile ahead: tile t's epilogue takes the slot of
        // tile t + 2 into s_q[t & 1], read after tile t + 1's main loop (main
        // loop barriers separate each write from the reads around it), so the
        // atomic's round trip hides behind the epilogue's own loads.
        __shared__ int s_slot, s_q[2];
        const int x = blockIdx.x & 7;
        const int tj_n = g.K / BN;                     // output [N, K] per expert
        const int tpe = (g.N / BM) * tj_n;
        const int tiles_x = min(max(sload(g.wg_cnt, x), 0), g.E) * tpe;
        int e = 0, i0 = 0, n0 = 0, nk = 0;
        // slot: wave-uniform; the lists are read through the scalar cache
        auto setup = [&](int slot) {
            const int eo = slot / tpe;
            const int tt = slot - eo * tpe;
            e = min(max(sload(g.wg_list, x * g.E + eo), 0), g.E - 1);
            i0 = (tt / tj_n) * BM;
            n0 = (tt - (tt / tj_n) * tj_n) * BN;
            const int64_t rb = sload(g.offsets, e);
            const int me = (int)(min((int64_t)sload(g.offsets, e + 1), g.R) - rb);
            nk = (me + BK - 1) / BK;
            // bounded to the expert's rows: the last reduction step's tail reads zeros
            la.init(make_rsrc_words(g.A + rb * g.lda + i0, (int64_t)me * g.lda * 2 - i0 * 2), g.lda);
            lb.init(make_rsrc_words(g.B + rb * g.ldb + n0, (int64_t)me * g.ldb * 2 - n0 * 2), g.ldb);
        };
        if (threadIdx.x == 0) {
            s_slot = atomicAdd(g.wg_ctr + x, 1);
            s_q[1] = atomicAdd(g.wg_ctr + x, 1);       // tile 1's slot, read after tile 0's main loop
        }
        __syncthreads();
        const int slot = __builtin_amdgcn_readfirstlane(s_slot);
        if (slot < 0 || slot >= tiles_x) return;
        // The next tile's first PRE steps go into stages [0, PRE) during this
        // tile's epilogue; the fused epilogue's weights go
        // through the stages after them (of A for waves 0-3, of B for waves
        // 4-7), two 4-KB slots per wave.
        // (without that epilogue the whole prologue, S-1 steps)
        constexpr int SLOT_STAGES = (4 * 8192 + A_BYTES - 1) / A_BYTES;
        constexpr bool LDS_EPI = WTN == 2 && WTM >= 2 && NW == 8 && S > SLOT_STAGES && A_BYTES == B_BYTES;
        constexpr int PRE = LDS_EPI ? S - SLOT_STAGES : S - 1;
        setup(slot);
        issue_steps(nk, 0, PRE - 1);
        const int wu = wave_id();                     // wave-uniform: LDS base and resource
        lds_t* wslots = wu < 4 ? smem + PRE * A_BYTES + wu * 8192
                               : smem + S * A_BYTES + PRE * B_BYTES + (wu - 4) * 8192;
        WStage ws;
        for (int tcount = 0;; ++tcount) {
            zero_acc();
            if constexpr (PP) mainloop_pp(nk, PRE, WTM, no_hook, no_hook);
            else mainloop(nk, PRE, no_hook);
            __syncthreads();          // LDS stages free; s_q[(tcount - 1) & 1] written before the main loop
            const int next = __builtin_amdgcn_readfirstlane(s_q[(tcount - 1) & 1]);
            const bool more = next >= 0 && next < tiles_x;
            int after = 0;
            if (threadIdx.x == 0 && more) after = atomicAdd(g.wg_ctr + x, 1);
            const int ce = e, ci0 = i0, cn0 = n0;
            // With the weights staged through LDS the epilogue's own loads go
            // first; the next tile's set-up loads overlap them, and its first
            // steps are issued once they have landed.
            const bool late = LDS_EPI && g.sg.out;
            if (more && !late) {
                setup(next);
                issue_steps(nk, 0, PRE - 1);
            }
            if (g.sg.out) {
                const int iw = ci0 + wm * 32 * WTM, jw = cn0 + wn * 32 * WTN;
                auto lds_epi = [&](auto kind_c) {
                    constexpr int KIND = decltype(kind_c)::value;
                    // the wave's first two weight slices (its other two are
                    // loaded as the first two are reduced)
                    ws.init(g.sg.W + ((int64_t)ce * g.N + ci0 + (wu / WVN) * 32 * WTM) * g.K + cn0 +
                                (wu % WVN) * 32 * WTN,
                            g.K, 32 * WTM);
                    ws.issue(wslots, 0);
                    ws.issue(wslots + 4096, 1);
                    SgEpiLds<KIND, WTM, WTN> ep;
                    ep.begin(g, ce, iw, jw, lane);
                    if (more) setup(next);
                    ep.template run<LOADS>(g, acc, ce, iw, jw, lane, ws, wslots, 0, [&]() {
                        if (more) issue_steps(nk, 0, PRE - 1);
                    });
                };
                if constexpr (LDS_EPI) {
                    if (g.sg.q.kind == K_NVFP4) lds_epi(std::integral_constant<int, K_NVFP4>{});
                    else if (g.sg.q.kind == K_INT) lds_epi(std::integral_constant<int, K_INT>{});
                    else lds_epi(std::integral_constant<int, K_FP8>{});
                } else {
                    if (g.sg.q.kind == K_NVFP4) sg_epilogue<K_NVFP4, WTM, WTN>(g, acc, ce, iw, jw, lane);
                    else if (g.sg.q.kind == K_INT) sg_epilogue<K_INT, WTM, WTN>(g, acc, ce, iw, jw, lane);
                    else sg_epilogue<K_FP8, WTM, WTN>(g, acc, ce, iw, jw, lane);
                }
            } else {
#pragma unroll
                for (int ti = 0; ti < WTM; ++ti) {
                    const int ml = wm * 32 * WTM + ti * 32 + (lane & 31);
#pragma unroll
                    for (int tj = 0; tj < WTN; ++tj) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int nl = wn * 32 * WTN + tj * 32 + 8 * q + 4 * (lane >> 5);
                            float* C = static_cast<float*>(g.C) + (int64_t)ce * g.strideC +
                                       (int64_t)(ci0 + ml) * g.ldc + cn0 + nl;
                            *reinterpret_cast<float4*>(C) = make_float4(acc[ti][tj][4 * q], acc[ti][tj][4 * q + 1],
                                                                        acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]);
                        }
                    }
                }
            }
            if (threadIdx.x == 0 && more) s_q[tcount & 1] = after;
            if (!more) break;
        }
        // nothing direct-to-LDS may be in flight when the block's LDS is released
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

// Large tile: 256 x 256 outputs, as WVM_BIG x WVN_BIG waves of
// (256 / WVM_BIG) x (256 / WVN_BIG); small tile: 128 x 128, 2 x 2 waves.
constexpr int BK_BIG = GEMM_BK_BIG, S_BIG = GEMM_S_BIG, BK_SMALL = 32, S_SMALL = 3;
constexpr int BK_WG = GEMM_BK_WG, S_WG = GEMM_S_WG;
constexpr int WVM_BIG = GEMM_WVM, WVN_BIG = GEMM_WVN;
#ifdef GEMM_WTM
constexpr int WTM_BIG = GEMM_WTM, WTN_BIG = GEMM_WTN;
#else
constexpr int WTM_BIG = 8 / WVM_BIG, WTN_BIG = 8 / WVN_BIG;
#endif
constexpr int BM_BIG = 32 * WTM_BIG * WVM_BIG, BN_BIG = 32 * WTN_BIG * WVN_BIG;
static_assert(BM_BIG == 256, "the large row tile is the 256-row tile table");
#define FQ_BIG(MODE) \
    k_gemm<MODE, WVM_BIG, WVN_BIG, WTM_BIG, WTN_BIG, MODE == WGRAD ? BK_WG : BK_BIG, MODE == WGRAD ? S_WG : S_BIG>
#define FQ_SMALL(MODE) k_gemm<MODE, 2, 2, 2, 2, BK_SMALL, S_SMALL>

// Explicit instantiations: without them the host pass does not emit every
// launch stub for this template.
template __global__ void FQ_BIG(FWD)(GemmArgs);
template __global__ void FQ_SMALL(FWD)(GemmArgs);
template __global__ void FQ_BIG(DGRAD)(GemmArgs);
template __global__ void FQ_SMALL(DGRAD)(GemmArgs);
template __global__ void FQ_BIG(WGRAD)(GemmArgs);
template __global__ void FQ_SMALL(WGRAD)(GemmArgs);

// Large tiles where the shapes allow, 128 x 128 otherwise.
template <int MODE>
hipError_t launch(const GemmArgs& g, hipStream_t st) {
    const bool big_m = MODE == WGRAD ? (g.N % BM_BIG == 0) : true;
    const bool big_n = (MODE == WGRAD ? g.K : g.N) % BN_BIG == 0;
    const int big = (big_m && big_n) ? 1 : 0;
    GemmArgs a = g;
    int64_t blocks;
    if (MODE != WGRAD) {
        if (g.R == 0) return hipSuccess;
        a.tile_expert = g.tables[big].tile_expert;
        a.tile_row0 = g.tables[big].tile_row0;
        a.num_tiles = g.tables[big].num_tiles;
        const int bm = big ? BM_BIG : 128, bn = big ? BN_BIG : 128;
        blocks = max_mtiles(g.R, g.E, bm) * (g.N / bn);
    } else {
        // persistent: as many blocks as are resident on the device at once
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err == hipSuccess)
            err = big ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, FQ_BIG(MODE), 64 * WVM_BIG * WVN_BIG, 0)
                      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, FQ_SMALL(MODE), 256, 0);
        if (err != hipSuccess) return err;
        blocks = (int64_t)(cus > 8 ? cus : 8) * (per_cu > 1 ? per_cu : 1);
    }
    blocks = (blocks + 7) / 8 * 8;       // a whole number of blocks per XCD
    if (big) hipLaunchKernelGGL((FQ_BIG(MODE)), dim3((unsigned)blocks), dim3(64 * WVM_BIG * WVN_BIG), 0, st, a);
    else hipLaunchKernelGGL((FQ_SMALL(MODE)), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// out[o] = sum of `per` consecutive partials (fixed order), o < n_out
// lanes per output of k_sg_sum: one for a few partials (a thread reads its
// run of <= 16 floats), else the power of two >= per, at most 64
__host__ __device__ __forceinline__ int sg_sum_lanes(int per) {
    int L = 1;
    if (per > 16)
        while (L < per && L < 64) L <<= 1;
    return L;
}

// out[o] = sum of part[o * per .. o * per + per): L lanes per output read its
// partials coalesced, lane j taking j, j + L, ..., then a fixed xor tree over
// the L lanes (deterministic)
__global__ __launch_bounds__(256) void k_sg_sum(const float* part, int64_t n_out, int per, float* out) {
    const int L = sg_sum_lanes(per);
    const int lane = threadIdx.x & 63;
    const int64_t o = ((int64_t)blockIdx.x * 256 + threadIdx.x) / L;
    const int j0 = lane & (L - 1);
    float acc = 0.0f;
    if (o < n_out) {
        const float* p = part + o * per;
        for (int i = j0; i < per; i += L) acc += p[i];
    }
    acc = group_sum(acc, L);
    if (o < n_out && j0 == 0) out[o] = acc;
}

// out[b] = sum over rows of in[b, :] (per-matrix gradient), fixed order
__global__ __launch_bounds__(256) void k_sg_batch(const float* in, int64_t rows, float* out) {
    __shared__ float red[256];
    const int64_t b = blockIdx.x;
    float acc = 0.0f;
    for (int64_t r = threadIdx.x; r < rows; r += 256) acc += in[b * rows + r];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[b] = red[0];
}

__global__ void k_zero_i32(int32_t* p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t st) {
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, st, p, n);
    return hipGetLastError();
}

// blocks of k_sg_sum for n_out outputs of `per` partials each
static unsigned sg_sum_blocks(int64_t n_out, int per) {
    return (unsigned)((n_out * sg_sum_lanes(per) + 255) / 256);
}

int sg_mode(const QParams& q) {
    if (q.kind == K_NONE || q.source == S_DYNAMIC) return 0;
    if (q.kind == K_NVFP4) return 1;
    if (q.gran == G_GROUP) return q.group == 16 ? 1 : (q.group >= 32 ? 2 : 0);
    return 2;
}

hipError_t launch_sg_reduce(const QParams& q, const float* part, int64_t E, int64_t N, int64_t K,
                            float* rowpart, float* out, hipStream_t st) {
    const int64_t rows = E * N, np = K / 32;
    if (q.gran == G_GROUP) {
        const int64_t n_out = rows * (K / q.group);
        hipLaunchKernelGGL(k_sg_sum, dim3(sg_sum_blocks(n_out, q.group / 32)), dim3(256), 0, st, part, n_out,
                           q.group / 32, out);
    } else if (q.gran == G_ROW) {
        hipLaunchKernelGGL(k_sg_sum, dim3(sg_sum_blocks(rows, (int)np)), dim3(256), 0, st, part, rows,
                           (int)np, out);
    } else {
        hipLaunchKernelGGL(k_sg_sum, dim3(sg_sum_blocks(rows, (int)np)), dim3(256), 0, st, part, rows,
                           (int)np, rowpart);
        hipLaunchKernelGGL(k_sg_batch, dim3((unsigned)E), dim3(256), 0, st, rowpart, N, out);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_fwd(const GemmArgs& g, hipStream_t st) { return launch<FWD>(g, st); }
hipError_t launch_gemm_dgrad(const GemmArgs& g, hipStream_t st) { return launch<DGRAD>(g, st); }
hipError_t launch_gemm_wgrad(const GemmArgs& g, hipStream_t st) { return launch<WGRAD>(g, st); }

}  // namespace fq
