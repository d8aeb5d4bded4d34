// Scale optimiser step: AdamW over the learnable quantiser scales, all
// gradients clipped by their global L2 norm (the optim settings of the
// AngelSlim "MCoreQAD Backend" page, "Train from YAML": lr 2e-4, weight decay
// 0, betas (0.9, 0.95), grad clip 1.0; nxmr.cn article, section 四).
//
// Three launches, none with atomics, so the step is bitwise deterministic:
//   k_adam_sq      block b sums g^2 (double) over a fixed run of ADAM_CHUNK
//                  elements of one tensor, then a fixed tree -> part[b];
//   k_adam_norm    one block: the partials in a fixed order -> norm, and the
//                  clip factor min(1, max_norm / (norm + 1e-6));
//   k_adam_update  elementwise, fp32:
//                    g' = g c;  m = b1 m + (1 - b1) g';  v = b2 v + (1 - b2) g'^2
//                    p = p (1 - lr wd) - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
//                  then the scale is clamped into its usable range: an NVFP4
//                  block scale into [t 2^-9, t 448] of its tensor scale t (a
//                  finite, non-zero E4M3 value of s / t), any other scale to
//                  >= 2^-126.
// Tensors whose four arrays are 16-B aligned with a length (and, projected,
// a tensor-scale run) divisible by 4 move 4 elements per lane per access; the
// rest go element by element.  The passes are HBM bound: 4 B per element for
// the norm, 28 B for the update.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int OPT_TPB = 256;

// fixed order: a wave xor-tree, then the waves' sums in wave order
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
    for (int m = 1; m < WAVE; m <<= 1) v += __shfl_xor(v, m);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < OPT_TPB / WAVE; ++w) t += red[w];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(OPT_TPB) void k_adam_sq(AdamArgs a) {
    __shared__ double red[OPT_TPB];
    int i = 0;
    while (i + 1 < a.np && (int64_t)blockIdx.x >= a.prm[i + 1].blk0) ++i;
    const AdamParam& q = a.prm[i];
    const int64_t lo = ((int64_t)blockIdx.x - q.blk0) * ADAM_CHUNK;
    const int64_t hi = min(lo + ADAM_CHUNK, q.n);
    double acc = 0.0;
    if (q.vec) {
        // four independent 16-B loads in flight per thread, summed in order
        const float4* g4 = reinterpret_cast<const float4*>(q.g);
        int64_t k = lo / 4 + threadIdx.x;
        for (; k + 3 * OPT_TPB < hi / 4; k += 4 * OPT_TPB) {
            float4 g[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) g[u] = g4[k + u * OPT_TPB];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc += (double)g[u].x * g[u].x + (double)g[u].y * g[u].y + (double)g[u].z * g[u].z +
                       (double)g[u].w * g[u].w;
        }
        for (; k < hi / 4; k += OPT_TPB) {
            const float4 g = g4[k];
            acc += (double)g.x * g.x + (double)g.y * g.y + (double)g.z * g.z + (double)g.w * g.w;
        }
    } else {
        for (int64_t k = lo + threadIdx.x; k < hi; k += OPT_TPB) {
            const double g = q.g[k];
            acc += g * g;
        }
    }
    const double s = block_sum(acc, red);
    if (threadIdx.x == 0) a.part[blockIdx.x] = s;
}

__global__ __launch_bounds__(OPT_TPB) void k_adam_norm(AdamArgs a) {
    __shared__ double red[OPT_TPB];
    double acc = 0.0;
    for (int b = threadIdx.x; b < a.nb; b += OPT_TPB) acc += a.part[b];
    const double norm = sqrt(block_sum(acc, red));
    if (threadIdx.x == 0) {
        const double c = a.max_norm > 0.0 ? fmin(1.0, a.max_norm / (norm + 1.0e-6)) : 1.0;
        a.clip[0] = (float)c;
        if (a.norm_out) a.norm_out[0] = (float)norm;
    }
}

struct Upd {
    float b1, b2, omb1, omb2, eps, decay, step_size, bc2_sqrt, c;
    __device__ __forceinline__ void operator()(float& p, float& m, float& v, float g, int proj, float t) const {
        g = g * c;
        m = b1 * m + omb1 * g;
        v = b2 * v + omb2 * (g * g);
        const float denom = sqrtf(v) / bc2_sqrt + eps;
        p = p * decay - step_size * (m / denom);
        p = proj == 1 ? fminf(fmaxf(p, t * 0x1p-9f), t * 448.0f) : fmaxf(p, 0x1p-126f);
    }
};

// index of element i's tensor scale: 32-bit division where the index fits (a uniform branch)
__device__ __forceinline__ int64_t tindex(const AdamParam& q, int64_t i) {
    return q.n <= 0x7fffffff ? (int64_t)((uint32_t)i / (uint32_t)q.per_t) : i / q.per_t;
}

__global__ __launch_bounds__(OPT_TPB) void k_adam_update(AdamArgs a) {
    const AdamParam& q = a.prm[blockIdx.y];
    const Upd u{a.b1, a.b2, a.one_m_b1, a.one_m_b2, a.eps, a.decay, a.step_size, a.bc2_sqrt, a.clip[0]};
    const int64_t stride = (int64_t)gridDim.x * OPT_TPB;
    if (q.vec) {
        float4* p4 = reinterpret_cast<float4*>(q.p);
        float4* m4 = reinterpret_cast<float4*>(q.m);
        float4* v4 = reinterpret_cast<float4*>(q.v);
        const float4* g4 = reinterpret_cast<const float4*>(q.g);
        for (int64_t j = (int64_t)blockIdx.x * OPT_TPB + threadIdx.x; j < q.n / 4; j += stride) {
            float4 p = p4[j], m = m4[j], v = v4[j];
            const float4 g = g4[j];
            const float t = q.proj == 1 ? q.t[tindex(q, 4 * j)] : 0.0f;   // shared by the 4 (per_t % 4 == 0)
            u(p.x, m.x, v.x, g.x, q.proj, t);
            u(p.y, m.y, v.y, g.y, q.proj, t);
            u(p.z, m.z, v.z, g.z, q.proj, t);
            u(p.w, m.w, v.w, g.w, q.proj, t);
            m4[j] = m;
            v4[j] = v;
            p4[j] = p;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * OPT_TPB + threadIdx.x; i < q.n; i += stride) {
            float p = q.p[i], m = q.m[i], v = q.v[i];
            const float t = q.proj == 1 ? q.t[tindex(q, i)] : 0.0f;
            u(p, m, v, q.g[i], q.proj, t);
            q.m[i] = m;
            q.v[i] = v;
            q.p[i] = p;
        }
    }
}

}  // namespace

int64_t adam_norm_blocks(int64_t count) {
    const int64_t nb = (count + ADAM_CHUNK - 1) / ADAM_CHUNK;
    return nb < 1 ? 1 : nb;
}

hipError_t launch_scale_adamw(const AdamArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_adam_sq, dim3((unsigned)a.nb), dim3(OPT_TPB), 0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_adam_norm, dim3(1), dim3(OPT_TPB), 0, st, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    int64_t nmax = 1;
    for (int i = 0; i < a.np; ++i) {
        const int64_t w = a.prm[i].vec ? a.prm[i].n / 4 : a.prm[i].n;
        nmax = w > nmax ? w : nmax;
    }
    int64_t gx = (nmax + OPT_TPB - 1) / OPT_TPB;
    gx = gx > 8192 ? 8192 : gx;
    hipLaunchKernelGGL(k_adam_update, dim3((unsigned)gx, (unsigned)a.np), dim3(OPT_TPB), 0, st, a);
    return hipGetLastError();
}

}  // namespace fq
