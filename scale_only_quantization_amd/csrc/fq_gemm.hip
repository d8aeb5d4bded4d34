// bf16 grouped GEMM over all experts on the gfx950 matrix cores (the single
// grouped GEMM of the nxmr.cn article on MCoreQAD, section 二.4).
//
// Three operand layouts share one kernel body:
//   FWD    C[r, n]    = sum_k A[r, k] B_e[n, k]      A routed rows, B [N, K]   (bf16 out)
//   DGRAD  C[r, n]    = sum_k A[r, k] B_e[k, n]      B stored [K, N]           (bf16 out)
//   WGRAD  C_e[i, j]  = sum_r A[r, i] B[r, j]        rows r of expert e        (fp32 out)
// Tiles: 128 x 128 outputs x 64 reduction per step, 256 threads = 4 waves as
// 2 x 2, each wave 64 x 64 outputs = 2 x 2 v_mfma_f32_32x32x16_bf16.  Both
// operand tiles live in LDS as [128 rows][64 reduction] bf16 (128 B per row),
// the 16-byte chunk index XOR-swizzled with (row ^ row >> 3) & 7 so the MFMA
// fragment reads (32 rows, one chunk) and the transposing writes of
// MN-contiguous operands both spread over the banks.  Two LDS stages: the next
// tile's global loads are in flight while the current one is multiplied.
// FWD/DGRAD row tiles come from the device-side tile table (expert, first row)
// built by the routing scan, so no host read-back of the counts is needed;
// WGRAD visits experts in descending row count (longest reductions first).
#include <type_traits>

#include "fq_common.h"
#include "fq_internal.h"

namespace fq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = GEMM_BM;      // 128
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int TILE_BYTES = 128 * BK * 2;   // one operand tile, 16 KB

enum Mode { FWD = 0, DGRAD = 1, WGRAD = 2 };

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int ch) { return row * 128 + ((ch ^ swz(row)) << 4); }

// Operand whose reduction index is contiguous in memory: element (row, k) at
// base_row[row] + k.  Thread t moves rows t/8 + 32p (p < 4), 16-B chunk t%8.
struct KLoader {
    const uint16_t* rowp[4];
    uint4 reg[4];
    __device__ __forceinline__ void load(int k0) {
        const int ch = threadIdx.x & 7;
#pragma unroll
        for (int p = 0; p < 4; ++p) reg[p] = *reinterpret_cast<const uint4*>(rowp[p] + k0 + ch * 8);
    }
    __device__ __forceinline__ void store(char* lds) const {
        const int ch = threadIdx.x & 7;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = (threadIdx.x >> 3) + 32 * p;
            *reinterpret_cast<uint4*>(lds + lds_off(row, ch)) = reg[p];
        }
    }
};

// Operand whose row index is contiguous: element (row, k) at base[k*ld + row].
// Thread t reads 4 consecutive k rows (kg = t/16) of 8 consecutive rows
// (chunk t%16) and writes them transposed: 8 rows x 4 k = 8 ds_write_b64.
// k >= kmax reads as zero (end of an expert's rows).
struct MNLoader {
    const uint16_t* base;
    int64_t ld;
    int kmax;
    uint4 reg[4];
    __device__ __forceinline__ void load(int k0) {
        const int nc = threadIdx.x & 15, kg = threadIdx.x >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + kg * 4 + i;
            reg[i] = k < kmax ? *reinterpret_cast<const uint4*>(base + (int64_t)k * ld + nc * 8)
                              : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
        const int nc = threadIdx.x & 15, kg = threadIdx.x >> 4;
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&reg[0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&reg[1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&reg[2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&reg[3]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = nc * 8 + j;
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
            uint2 v;
            v.x = __builtin_amdgcn_perm(r1[j >> 1], r0[j >> 1], sel);
            v.y = __builtin_amdgcn_perm(r3[j >> 1], r2[j >> 1], sel);
            *reinterpret_cast<uint2*>(lds + lds_off(row, kg >> 1) + (kg & 1) * 8) = v;
        }
    }
};

template <int MODE>
__global__ __launch_bounds__(NT) void k_gemm(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char smem[2][2][TILE_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int e, nk;
    int64_t m0 = 0, m_end = 0;      // FWD/DGRAD: routed row range of the tile's expert
    int n0, i0 = 0;
    typedef typename std::conditional<MODE == WGRAD, MNLoader, KLoader>::type ALoad;
    typedef typename std::conditional<MODE == FWD, KLoader, MNLoader>::type BLoad;
    ALoad la;
    BLoad lb;

    if (MODE != WGRAD) {
        const int ntn = g.N / BN;
        const int mt = blockIdx.x / ntn;
        const int nt = blockIdx.x - mt * ntn;
        if (mt >= g.num_tiles[0]) return;
        e = min(max(g.tile_expert[mt], 0), g.E - 1);
        m0 = g.tile_row0[mt];
        m_end = min((int64_t)g.offsets[e + 1], g.R);
        n0 = nt * BN;
        nk = g.K / BK;
        const int ch_row = tid >> 3;
        if constexpr (MODE != WGRAD) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                int64_t r = m0 + ch_row + 32 * p;
                if (r > g.R - 1) r = g.R - 1;
                la.rowp[p] = g.A + r * g.lda;
            }
        }
        const uint16_t* Be = g.B + (int64_t)e * g.strideB;
        if constexpr (MODE == FWD) {
#pragma unroll
            for (int p = 0; p < 4; ++p) lb.rowp[p] = Be + (int64_t)(n0 + ch_row + 32 * p) * g.ldb;
        } else if constexpr (MODE == DGRAD) {
            lb.base = Be + n0;
            lb.ld = g.ldb;
            lb.kmax = g.K;
        }
    } else {
        const int tj = g.K / BN;              // output [N, K] per expert
        const int tpe = (g.N / BM) * tj;
        const int eo = blockIdx.x / tpe;
        const int tt = blockIdx.x - eo * tpe;
        e = min(max(g.order[eo], 0), g.E - 1);
        i0 = (tt / tj) * BM;
        n0 = (tt - (tt / tj) * tj) * BN;
        const int64_t rb = g.offsets[e];
        const int me = (int)(min((int64_t)g.offsets[e + 1], g.R) - rb);
        nk = (me + BK - 1) / BK;
        if constexpr (MODE == WGRAD) {
            la.base = g.A + rb * g.lda + i0;
            la.ld = g.lda;
            la.kmax = me;
            lb.base = g.B + rb * g.ldb + n0;
            lb.ld = g.ldb;
            lb.kmax = me;
        }
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    if (nk > 0) {
        la.load(0);
        lb.load(0);
        la.store(smem[0][0]);
        lb.store(smem[0][1]);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            la.load((kt + 1) * BK);
            lb.load((kt + 1) * BK);
        }
        const char* sa = smem[cur][0];
        const char* sb = smem[cur][1];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = kk * 2 + (lane >> 5);
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = *reinterpret_cast<const bf16x8*>(sa + lds_off(wm * 64 + t * 32 + (lane & 31), ch));
                bfr[t] = *reinterpret_cast<const bf16x8*>(sb + lds_off(wn * 64 + t * 32 + (lane & 31), ch));
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
                    acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[tj], af[ti], acc[ti][tj], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            la.store(smem[cur ^ 1][0]);
            lb.store(smem[cur ^ 1][1]);
        }
        __syncthreads();
    }

    // epilogue: lane holds C[m = lane%32][n = 8*(v/4) + 4*(lane/32) + v%4] of each 32x32 tile
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int ml = wm * 64 + ti * 32 + (lane & 31);
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * 64 + tj * 32 + 8 * q + 4 * (lane >> 5);
                const float c0 = acc[ti][tj][4 * q], c1 = acc[ti][tj][4 * q + 1];
                const float c2 = acc[ti][tj][4 * q + 2], c3 = acc[ti][tj][4 * q + 3];
                if (MODE == WGRAD) {
                    float* C = static_cast<float*>(g.C) + (int64_t)e * g.strideC +
                               (int64_t)(i0 + ml) * g.ldc + n0 + nl;
                    *reinterpret_cast<float4*>(C) = make_float4(c0, c1, c2, c3);
                } else {
                    const int64_t r = m0 + ml;
                    if (r < m_end) {
                        uint16_t* C = static_cast<uint16_t*>(g.C) + r * g.ldc + n0 + nl;
                        *reinterpret_cast<uint2*>(C) = make_uint2(pack_bf16(c0, c1), pack_bf16(c2, c3));
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_fwd(const GemmArgs& g, hipStream_t st) {
    if (g.R == 0) return hipSuccess;
    const int64_t blocks = max_mtiles(g.R, g.E) * (g.N / BN);
    hipLaunchKernelGGL(k_gemm<FWD>, dim3((unsigned)blocks), dim3(NT), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_gemm_dgrad(const GemmArgs& g, hipStream_t st) {
    if (g.R == 0) return hipSuccess;
    const int64_t blocks = max_mtiles(g.R, g.E) * (g.N / BN);
    hipLaunchKernelGGL(k_gemm<DGRAD>, dim3((unsigned)blocks), dim3(NT), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_gemm_wgrad(const GemmArgs& g, hipStream_t st) {
    const int64_t blocks = (int64_t)g.E * (g.N / BM) * (g.K / BN);
    hipLaunchKernelGGL(k_gemm<WGRAD>, dim3((unsigned)blocks), dim3(NT), 0, st, g);
    return hipGetLastError();
}

}  // namespace fq
