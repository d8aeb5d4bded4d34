// Self-distillation losses on logits (the nxmr.cn article, section 二.5:
// total = lm_weight lm_loss + distill_weight distill_loss; distill_type kl,
// rkl or cakld; distill_topk > 0 restricts the KL to the teacher's top-k
// tokens).  One 1024-thread block per token row, two passes over the row, no
// atomics:
//   pass 1  online (max, sum of exp) of the student's and the teacher's
//           logits, with the sums the losses need:
//             A = sum e^{zt - mt} (zt - zs)   -> kl  = A / St + lse_s - lse_t
//             B = sum e^{zs - ms} (zs - zt)   -> rkl = B / Ss + lse_t - lse_s
//           the teacher's confidence is 1 / St (its largest probability);
//           the sums run in base 2 (the frame m log2 e, one fused
//           multiply-add per exponent);
//           a fixed tree combines the threads' partial states.
//   pass 2  d loss / d zs per element (q = e^{zs - lse_s}, p = e^{zt - lse_t}):
//             kl  q - p;  rkl  q ((zs - lse_s) - (zt - lse_t) - rkl);
//             cakld  c (q - p) + (1 - c) rkl-term;  top-k kl  q - p~ on the k ids;
//             LM  q - [v == label];  all times 1 / T, then bf16.
//           The label and the top-k ids are rewritten after a barrier by one
//           wave, from the inputs, so each element is rounded once.
// Per row: 4 B (kl/rkl/cakld: 2 x bf16 logits) read per element per pass and
// 2 B written.  With the teacher's logits the four exponentials per element
// keep the kernel near the vector issue rate; top-k (one input) is bound by
// its loads, so each thread keeps DU vectors' loads in flight.
#include <hip/hip_runtime.h>

#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int DTPB = 1024;
constexpr int DWAVES = DTPB / WAVE;

// a token id from the caller, kept inside the row (ids are a precondition)
__device__ __forceinline__ int clamp_id(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }
__device__ __forceinline__ float bf_from_bits(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

constexpr float LOG2E = 0x1.715476p+0f;   // log2(e) and ln(2), rounded to fp32
constexpr float LN2 = 0x1.62e430p-1f;
// 2^x with the hardware exponential (a few ulp; results below the normal
// range may flush to zero, which the sums here cannot notice)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Keeps the block it stands in behind a branch: the compiler would otherwise
// evaluate a short conditional block (a rescale: one exponential, two
// products) on every pass and select, where a skipped branch costs a few
// scalar instructions once no lane's maximum rises any more.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }

// Running sums in base 2: the frame m is fl(max x * log2 e), s = sum of
// 2^{x log2 e - m} (each exponent one fused multiply-add), and a weighted sum
// in the same frame.  Ratios of the sums do not depend on the frame; the log
// of the sum of e^x is m ln 2 + ln s.
struct OnlineSum {
    float m = -INFINITY, s = 0.0f, a = 0.0f;
    __device__ __forceinline__ void merge(float m2, float s2, float a2) {
        const float mm = fmaxf(m, m2);
        if (mm == -INFINITY) return;
        const float f1 = m == -INFINITY ? 0.0f : exp2_hw(m - mm);
        const float f2 = m2 == -INFINITY ? 0.0f : exp2_hw(m2 - mm);
        s = s * f1 + s2 * f2;
        a = a * f1 + a2 * f2;
        m = mm;
    }
};

__device__ __forceinline__ void wave_merge(OnlineSum& o) {
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const float m2 = __shfl_xor(o.m, d), s2 = __shfl_xor(o.s, d), a2 = __shfl_xor(o.a, d);
        o.merge(m2, s2, a2);
    }
}

// block-wide merge of two online sums in a fixed order; every thread gets the result
__device__ __forceinline__ void block_merge(OnlineSum& o1, OnlineSum& o2, float* red) {
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    wave_merge(o1);
    wave_merge(o2);
    if (lane == 0) {
        red[w * 6 + 0] = o1.m; red[w * 6 + 1] = o1.s; red[w * 6 + 2] = o1.a;
        red[w * 6 + 3] = o2.m; red[w * 6 + 4] = o2.s; red[w * 6 + 5] = o2.a;
    }
    __syncthreads();
    OnlineSum r1, r2;
    for (int i = 0; i < DWAVES; ++i) {
        r1.merge(red[i * 6 + 0], red[i * 6 + 1], red[i * 6 + 2]);
        r2.merge(red[i * 6 + 3], red[i * 6 + 4], red[i * 6 + 5]);
    }
    __syncthreads();
    o1 = r1;
    o2 = r2;
}

// DU vectors of 8 logits per thread in flight: the row's vectors v0,
// v0 + DTPB, ... (zero past the row's end) of the student and, with TEACHER,
// the teacher
constexpr int DU = 4;
template <bool TEACHER>
__device__ __forceinline__ void load_vecs(const uint4* zs, const uint4* zt, int v0, int nvec, uint4* bs,
                                          uint4* bt) {
#pragma unroll
    for (int u = 0; u < DU; ++u) {
        const int v = v0 + u * DTPB;
        bs[u] = bt[u] = make_uint4(0, 0, 0, 0);
        if (v < nvec) {
            bs[u] = zs[v];
            if (TEACHER) bt[u] = zt[v];
        }
    }
}

template <int KIND>
__global__ __launch_bounds__(DTPB) void k_distill(DistillArgs a) {
    __shared__ float red[DWAVES * 6];
    __shared__ float s_lpt[64];          // the teacher's top-k log-probabilities (renormalised)
    const int nvec = (int)(a.V >> 3);
    for (int64_t r = blockIdx.x; r < a.T; r += gridDim.x) {
        const uint4* zs = reinterpret_cast<const uint4*>(a.zs + r * a.V);
        const uint4* zt = reinterpret_cast<const uint4*>(a.zt + r * a.V);
        // ---- pass 1
        OnlineSum st_, ss_;              // teacher (with A), student (with B)
        // DU vectors' loads per thread go out before any is summed; they are
        // taken in the order of one at a time (v, v + DTPB, ...), so the sums
        // are the same
        for (int v0 = threadIdx.x; v0 < nvec; v0 += DU * DTPB) {
            uint4 bs[DU], bt[DU];
            load_vecs<KIND != DK_TOPK>(zs, zt, v0, nvec, bs, bt);
#pragma unroll
            for (int u = 0; u < DU; ++u) {
                if (v0 + u * DTPB >= nvec) break;
                float fs[8], ft[8], dts[8];      // dts = zt - zs
                unpack8(bs[u], fs);
                float mv = fs[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) mv = fmaxf(mv, fs[i]);
                // running sums rescaled only when the vector raises the running max
                if (KIND != DK_TOPK) {
                    unpack8(bt[u], ft);
                    float mt = ft[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, ft[i]);
                    mt *= LOG2E;
                    if (mt > st_.m) {
                        keep_branch();
                        const float f = exp2_hw(st_.m - mt);
                        st_.s *= f;
                        st_.a *= f;
                        st_.m = mt;
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float e = exp2_hw(__builtin_fmaf(ft[i], LOG2E, -st_.m));
                        st_.s += e;
                        dts[i] = ft[i] - fs[i];
                        st_.a = __builtin_fmaf(e, dts[i], st_.a);
                    }
                }
                mv *= LOG2E;
                if (mv > ss_.m) {
                    keep_branch();
                    const float f = exp2_hw(ss_.m - mv);
                    ss_.s *= f;
                    ss_.a *= f;
                    ss_.m = mv;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e = exp2_hw(__builtin_fmaf(fs[i], LOG2E, -ss_.m));
                    ss_.s += e;
                    if (KIND == DK_RKL || KIND == DK_CAKLD) ss_.a = __builtin_fmaf(-e, dts[i], ss_.a);
                }
            }
        }
        block_merge(st_, ss_, red);
        const float lse_s = __builtin_fmaf(ss_.m, LN2, __logf(ss_.s));
        float lse_t = 0.0f, kl = 0.0f, rkl = 0.0f, conf = 1.0f;
        if (KIND != DK_TOPK) {
            lse_t = __builtin_fmaf(st_.m, LN2, __logf(st_.s));
            kl = st_.a / st_.s + lse_s - lse_t;
            rkl = ss_.a / ss_.s + lse_t - lse_s;
            conf = 1.0f / st_.s;
        }
        // ---- the row's loss: one wave (top-k terms, label)
        float kd = KIND == DK_KL ? kl : KIND == DK_RKL ? rkl : conf * kl + (1.0f - conf) * rkl;
        if (threadIdx.x < WAVE) {
            const int lane = threadIdx.x;
            if (KIND == DK_TOPK) {
                const float tv = lane < a.k ? a.top_v[r * a.k + lane] : -INFINITY;
                const float tm = wave_max(tv);
                const float te = lane < a.k ? __expf(tv - tm) : 0.0f;
                const float tl = tm + __logf(wave_sum(te));
                const float lpt = tv - tl;                      // log p~
                const int id = lane < a.k ? clamp_id(a.top_i[r * a.k + lane], (int)a.V) : 0;
                const float lq = lane < a.k ? bf_from_bits(a.zs[r * a.V + id]) - lse_s : 0.0f;
                kd = wave_sum(lane < a.k ? __expf(lpt) * (lpt - lq) : 0.0f);
                if (lane < a.k) s_lpt[lane] = lpt;
            }
            if (lane == 0) {
                float row = a.dist_w * kd;
                if (a.labels) {
                    const int lab = clamp_id(a.labels[r], (int)a.V);
                    row += a.lm_w * (lse_s - bf_from_bits(a.zs[r * a.V + lab]));
                }
                a.row_loss[r] = row;
            }
        }
        if (!a.grad) {
            __syncthreads();
            continue;
        }
        // ---- pass 2
        uint4* g = reinterpret_cast<uint4*>(a.grad + r * a.V);
        const float ws = a.inv_T * (a.labels ? a.lm_w : 0.0f), wd = a.inv_T * a.dist_w;
        // ws q + wd gk per kind, gathered in q and p with the row's constants
        // (d = (zs - zt) - (lse_s - lse_t + rkl) is the rkl-term's factor):
        //   kl     q (ws + wd) - wd p          rkl    q (ws + wd d)
        //   cakld  q (ws + wd c + wd (1 - c) d) - wd c p
        //   top-k  q (ws + wd)  (the k ids are rewritten below)
        const float lsL = lse_s * LOG2E, ltL = lse_t * LOG2E;
        const float c0 = (lse_s - lse_t) + rkl;
        const float k1 = KIND == DK_RKL ? ws : KIND == DK_CAKLD ? ws + wd * conf : ws + wd;
        const float k2 = KIND == DK_RKL ? wd : wd * (1.0f - conf);
        const float k3 = KIND == DK_KL ? wd : wd * conf;
        for (int v0 = threadIdx.x; v0 < nvec; v0 += DU * DTPB) {
            uint4 bs[DU], bt[DU];
            load_vecs<KIND != DK_TOPK>(zs, zt, v0, nvec, bs, bt);
#pragma unroll
            for (int u = 0; u < DU; ++u) {
                if (v0 + u * DTPB >= nvec) break;
                float fs[8], ft[8], o[8];
                unpack8(bs[u], fs);
                if (KIND != DK_TOPK) unpack8(bt[u], ft);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float q = exp2_hw(__builtin_fmaf(fs[i], LOG2E, -lsL));
                    if (KIND == DK_TOPK) {
                        o[i] = q * k1;
                    } else {
                        const float p = exp2_hw(__builtin_fmaf(ft[i], LOG2E, -ltL));
                        const float d = (fs[i] - ft[i]) - c0;
                        if (KIND == DK_KL) o[i] = __builtin_fmaf(q, k1, -k3 * p);
                        else if (KIND == DK_RKL) o[i] = q * __builtin_fmaf(k2, d, k1);
                        else o[i] = __builtin_fmaf(q, __builtin_fmaf(k2, d, k1), -k3 * p);
                    }
                }
                g[v0 + u * DTPB] = pack8(o);
            }
        }
        __syncthreads();                 // every element written before the special ones are rewritten
        if (threadIdx.x < WAVE) {
            const int lane = threadIdx.x;
            const int lab = a.labels ? clamp_id(a.labels[r], (int)a.V) : -1;
            // d loss / d zs at one element, from the inputs (pt: p~ there, or 0)
            auto exact = [&](int id, float pt) {
                const float lq = bf_from_bits(a.zs[r * a.V + id]) - lse_s;
                const float q = __expf(lq);
                float gk = q - pt;
                if (KIND != DK_TOPK) {
                    const float lp = bf_from_bits(a.zt[r * a.V + id]) - lse_t;
                    const float p = __expf(lp);
                    const float gr = q * ((lq - lp) - rkl);
                    gk = KIND == DK_KL ? q - p : KIND == DK_RKL ? gr : conf * (q - p) + (1.0f - conf) * gr;
                }
                return bf16_bits(ws * (q - (id == lab ? 1.0f : 0.0f)) + wd * gk);
            };
            bool lab_done = false;
            if (KIND == DK_TOPK) {                   // the k top-k ids, one per lane
                const int id = lane < a.k ? clamp_id(a.top_i[r * a.k + lane], (int)a.V) : -1;
                if (id >= 0) a.grad[r * a.V + id] = exact(id, __expf(s_lpt[lane]));
                lab_done = __any(id >= 0 && id == lab);
            }
            if (lane == 0 && lab >= 0 && !lab_done) a.grad[r * a.V + lab] = exact(lab, 0.0f);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void k_row_mean(const float* rows, int64_t T, float inv_T, float* out) {
    __shared__ double red[256];
    double acc = 0.0;
    for (int64_t r = threadIdx.x; r < T; r += 256) acc += rows[r];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = (float)(red[0] * (double)inv_T);
}

}  // namespace

hipError_t launch_distill(const DistillArgs& a, float* mean_out, hipStream_t st) {
    if (a.T > 0) {
        int dev = 0, cus = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        // one row in flight per CU: the rows in flight (256 x 608 KB at the Qwen3
        // vocabulary) then fit the last-level cache, and pass 2 re-reads from it
        const int64_t grid = a.T < (int64_t)cus ? a.T : (int64_t)cus;
        switch (a.kind) {
        case DK_KL: hipLaunchKernelGGL(k_distill<DK_KL>, dim3((unsigned)grid), dim3(DTPB), 0, st, a); break;
        case DK_RKL: hipLaunchKernelGGL(k_distill<DK_RKL>, dim3((unsigned)grid), dim3(DTPB), 0, st, a); break;
        case DK_CAKLD: hipLaunchKernelGGL(k_distill<DK_CAKLD>, dim3((unsigned)grid), dim3(DTPB), 0, st, a); break;
        default: hipLaunchKernelGGL(k_distill<DK_TOPK>, dim3((unsigned)grid), dim3(DTPB), 0, st, a); break;
        }
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_row_mean, dim3(1), dim3(256), 0, st, a.row_loss, a.T, a.inv_T, mean_out);
    return hipGetLastError();
}

}  // namespace fq
