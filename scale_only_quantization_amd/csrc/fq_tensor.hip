// Fake-quant of one [batch, rows, cols] bf16 tensor along cols, forward and
// straight-through backward (the weight parametrisation / activation pre-hook
// of the nxmr.cn article on MCoreQAD, section 二.3, over a whole 3D expert
// stack at once, section 二.4).
//
// Layout: one wave64 per row; lane l handles 8 consecutive elements (one 16-byte
// load) at vector v = l, l + 64, ...  A 16-element NVFP4 block is a lane pair,
// a group of g elements is g/8 consecutive lanes, so every per-block value
// (block factor, dynamic amax, scale-gradient partial) is formed with lane
// shuffles inside the wave.  HBM-bound: 2 B (x) + 2 B (y) per element forward,
// 2 B + 2-4 B (grad) per element backward, plus the scales.
#include "fq_common.h"
#include "fq_internal.h"

namespace fq {

namespace {

constexpr int TPB = 256;            // 4 waves per block, one row per wave
constexpr int RPB = TPB / WAVE;

__device__ __forceinline__ float amax8(const float* f) {
    float m = fabsf(f[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

// Effective scale of the 8 elements of vector v of row `grow`, and the NVFP4
// block factor d (1 otherwise) and its E4M3 code.
template <int KIND, bool DYN, bool CODES = true>
__device__ __forceinline__ float vec_scale(const TensorArgs& a, int64_t grow, int64_t b, int v,
                                           const float* f, float row_s, float t,
                                           float* dfac, uint32_t* bcode) {
    *dfac = 1.0f;
    *bcode = 0;
    if (KIND == K_NVFP4) {
        float ratio;
        if (DYN) {
            float m = amax8(f);
            m = fmaxf(m, __shfl_xor(m, 1));                 // 16-element block = lane pair
            ratio = m / (6.0f * t);
        } else {
            ratio = a.scale[grow * (a.cols >> 4) + (v >> 1)] / t;
        }
        float d = CODES ? e4m3_round(fminf(ratio, 448.0f), bcode) : e4m3_round(fminf(ratio, 448.0f));
        *dfac = d;
        return t * d;
    }
    if (a.q.gran == G_GROUP) {
        const int gl = a.q.group >> 3;
        if (DYN) {
            float m = group_max(amax8(f), gl);
            return m / a.q.qdiv;
        }
        return a.scale[grow * (a.cols / a.q.group) + v / gl];
    }
    return row_s;
}

template <int KIND, bool DYN>
__device__ __forceinline__ float row_scale(const TensorArgs& a, int64_t grow, int64_t b, int lane,
                                           const uint4* xr, int nvec) {
    if (KIND == K_NVFP4) return 0.0f;
    if (DYN) {
        if (a.q.gran != G_ROW) return 0.0f;
        float m = 0.0f;
        for (int v = lane; v < nvec; v += WAVE) {
            float f[8];
            unpack8(xr[v], f);
            m = fmaxf(m, amax8(f));
        }
        return wave_max(m) / a.q.qdiv;
    }
    if (a.q.gran == G_ROW) return a.scale[grow];
    if (a.q.gran == G_TENSOR) return a.scale[b];
    return 0.0f;
}

// CODES: the 4/8-bit codes (and NVFP4 block-scale codes) are formed only when
// the caller asks for them; without them the per-element code logic is not
// compiled in
template <int KIND, bool DYN, bool CODES>
__global__ __launch_bounds__(TPB) void k_tensor_fwd(TensorArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t nrows = a.batch * a.rows;
    const int nvec = (int)(a.cols >> 3);
    const float qmin = a.q.qmin, qmax = a.q.qmax;
    const bool four_bit = (KIND == K_NVFP4) || (KIND == K_INT && qmax - qmin < 16.0f);
    for (int64_t grow = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6); grow < nrows;
         grow += (int64_t)gridDim.x * RPB) {
        const int64_t b = grow / a.rows;
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + grow * a.cols);
        const float row_s = row_scale<KIND, DYN>(a, grow, b, lane, xr, nvec);
        const float t = (KIND == K_NVFP4) ? a.tscale[b] : 0.0f;
        for (int v = lane; v < nvec; v += WAVE) {
            float f[8];
            unpack8(xr[v], f);
            float dfac;
            uint32_t bc;
            const float s = vec_scale<KIND, DYN, CODES>(a, grow, b, v, f, row_s, t, &dfac, &bc);
            float yv[8];
            uint32_t c4 = 0;
            uint32_t c8[2] = {0u, 0u};
            quant_group<KIND, 8>(f, s, qmin, qmax, [&](int i, const Elem& e) {
                yv[i] = e.q * s;
                if (CODES) {
                    const uint32_t c = elem_code<KIND>(e, f[i]);
                    c4 |= (c & 0xFu) << (4 * i);
                    c8[i >> 2] |= (c & 0xFFu) << (8 * (i & 3));
                }
            });
            if (a.y) reinterpret_cast<uint4*>(a.y + grow * a.cols)[v] = pack8(yv);
            if (CODES && a.codes) {
                if (four_bit)
                    reinterpret_cast<uint32_t*>(a.codes + grow * (a.cols >> 1))[v] = c4;
                else
                    reinterpret_cast<uint2*>(a.codes + grow * a.cols)[v] = make_uint2(c8[0], c8[1]);
            }
            if (CODES && KIND == K_NVFP4 && a.bcodes && !(v & 1))
                a.bcodes[grow * (a.cols >> 4) + (v >> 1)] = (uint8_t)bc;
        }
    }
}

__device__ __forceinline__ void load_grad8(const TensorArgs& a, int64_t grow, int v, float* g, int64_t gv = -1) {
    if (gv < 0) gv = grow * (a.cols >> 3) + v;             // flat vector index
    if (a.gy_fp32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.gy)) + 2 * gv;
        float4 u0 = p[0], u1 = p[1];
        g[0] = u0.x; g[1] = u0.y; g[2] = u0.z; g[3] = u0.w;
        g[4] = u1.x; g[5] = u1.y; g[6] = u1.z; g[7] = u1.w;
    } else {
        unpack8(reinterpret_cast<const uint4*>(a.gy)[gv], g);
    }
}

template <int KIND, bool DYN>
__global__ __launch_bounds__(TPB) void k_tensor_bwd(TensorArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t nrows = a.batch * a.rows;
    const int nvec = (int)(a.cols >> 3);
    const float qmin = a.q.qmin, qmax = a.q.qmax;
    // INT/FP8 dynamic: the scale is detached and the gradient passes straight
    constexpr bool PASS_ONLY = DYN && KIND != K_NVFP4;
    const bool per_row_sum = (KIND == K_NVFP4) ? DYN : (a.q.gran != G_GROUP);
    for (int64_t grow = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6); grow < nrows;
         grow += (int64_t)gridDim.x * RPB) {
        const int64_t b = grow / a.rows;
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + grow * a.cols);
        const float row_s = PASS_ONLY ? 0.0f : row_scale<KIND, DYN>(a, grow, b, lane, xr, nvec);
        const float t = (KIND == K_NVFP4) ? a.tscale[b] : 0.0f;
        float rowacc = 0.0f;
        for (int v = lane; v < nvec; v += WAVE) {
            float g[8];
            load_grad8(a, grow, v, g);
            if (PASS_ONLY) {
                if (a.gx) reinterpret_cast<uint4*>(a.gx + grow * a.cols)[v] = pack8(g);
                continue;
            }
            float f[8];
            unpack8(xr[v], f);
            float dfac;
            uint32_t bc;
            const float s = vec_scale<KIND, DYN, false>(a, grow, b, v, f, row_s, t, &dfac, &bc);
            float gx[8];
            float part = 0.0f;
            quant_group<KIND, 8>(f, s, qmin, qmax, [&](int i, const Elem& e) {
                const float c = ste_c(e, qmin, qmax);
                gx[i] = DYN ? g[i] : g[i] * (e.inside ? 1.0f : 0.0f);   // g * mask (signed zero)
                part = __builtin_fmaf(g[i], c, part);
            });
            if (a.gx) reinterpret_cast<uint4*>(a.gx + grow * a.cols)[v] = pack8(gx);
            if (a.gscale) {
                if (KIND == K_NVFP4) {
                    if (DYN) {
                        rowacc = __builtin_fmaf(part, dfac, rowacc);
                    } else {
                        const float tot = part + __shfl_xor(part, 1);
                        if (!(v & 1)) a.gscale[grow * (a.cols >> 4) + (v >> 1)] = tot;
                    }
                } else if (a.q.gran == G_GROUP) {
                    const int gl = a.q.group >> 3;
                    const float tot = group_sum(part, gl);
                    if ((lane & (gl - 1)) == 0) a.gscale[grow * (a.cols / a.q.group) + v / gl] = tot;
                } else {
                    rowacc += part;
                }
            }
        }
        if (!PASS_ONLY && a.gscale && per_row_sum) {
            const float tot = wave_sum(rowacc);
            if (lane == 0) {
                if (KIND != K_NVFP4 && a.q.gran == G_ROW) a.gscale[grow] = tot;
                else a.rowpart[grow] = tot;
            }
        }
    }
}

// Flat layout: one lane per 8-element vector of a matrix (blockIdx.y is the
// batch index), so that a wave reads and writes 1 KB contiguous whatever the
// row length (rows of 768 leave a row-per-wave kernel a quarter idle).  Used
// for NVFP4 block scales and per-group scales, whose index is the vector's
// flat index over 2 or group/8: blocks and groups align with lane pairs and
// lane groups because the row length is a multiple of the block or group.
template <int KIND, bool DYN, bool CODES = true>
__device__ __forceinline__ float flat_scale(const TensorArgs& a, int64_t gv, int sh, const float* f, float t,
                                            uint32_t* bc) {
    if (KIND == K_NVFP4) {
        float ratio;
        if (DYN) {
            float m = amax8(f);
            m = fmaxf(m, __shfl_xor(m, 1));                 // 16-element block = lane pair
            ratio = m / (6.0f * t);
        } else {
            ratio = a.scale[gv >> 1] / t;
        }
        if (!CODES) {
            *bc = 0;
            return t * e4m3_round(fminf(ratio, 448.0f));
        }
        return t * e4m3_round(fminf(ratio, 448.0f), bc);
    }
    *bc = 0;
    if (DYN) return group_max(amax8(f), a.q.group >> 3) / a.q.qdiv;
    return a.scale[gv >> sh];
}

template <int KIND, bool DYN, bool CODES>
__global__ __launch_bounds__(TPB) void k_tensor_fwd_flat(TensorArgs a) {
    const int64_t per = a.rows * (a.cols >> 3);             // vectors per matrix
    const int64_t b = blockIdx.y;
    const int sh = __builtin_ctz((unsigned)(a.q.group >> 3));   // group vectors = 2^sh
    const float qmin = a.q.qmin, qmax = a.q.qmax;
    const bool four_bit = (KIND == K_NVFP4) || (KIND == K_INT && qmax - qmin < 16.0f);
    const float t = (KIND == K_NVFP4) ? a.tscale[b] : 0.0f;
    for (int64_t gm = (int64_t)blockIdx.x * TPB + threadIdx.x; gm < per; gm += (int64_t)gridDim.x * TPB) {
        const int64_t gv = b * per + gm;
        float f[8];
        unpack8(reinterpret_cast<const uint4*>(a.x)[gv], f);
        uint32_t bc;
        const float s = flat_scale<KIND, DYN, CODES>(a, gv, sh, f, t, &bc);
        float yv[8];
        uint32_t c4 = 0;
        uint32_t c8[2] = {0u, 0u};
        quant_group<KIND, 8>(f, s, qmin, qmax, [&](int i, const Elem& e) {
            yv[i] = e.q * s;
            if (CODES) {
                const uint32_t c = elem_code<KIND>(e, f[i]);
                c4 |= (c & 0xFu) << (4 * i);
                c8[i >> 2] |= (c & 0xFFu) << (8 * (i & 3));
            }
        });
        if (a.y) reinterpret_cast<uint4*>(a.y)[gv] = pack8(yv);
        if (CODES && a.codes) {
            if (four_bit) reinterpret_cast<uint32_t*>(a.codes)[gv] = c4;
            else reinterpret_cast<uint2*>(a.codes)[gv] = make_uint2(c8[0], c8[1]);
        }
        if (CODES && KIND == K_NVFP4 && a.bcodes && !(gv & 1)) a.bcodes[gv >> 1] = (uint8_t)bc;
    }
}

template <int KIND, bool DYN>
__global__ __launch_bounds__(TPB) void k_tensor_bwd_flat(TensorArgs a) {
    const int64_t nvec_row = a.cols >> 3;
    const int64_t per = a.rows * nvec_row;
    const int64_t b = blockIdx.y;
    const int sh = __builtin_ctz((unsigned)(a.q.group >> 3));
    const float qmin = a.q.qmin, qmax = a.q.qmax;
    constexpr bool PASS_ONLY = DYN && KIND != K_NVFP4;
    const float t = (KIND == K_NVFP4) ? a.tscale[b] : 0.0f;
    for (int64_t gm = (int64_t)blockIdx.x * TPB + threadIdx.x; gm < per; gm += (int64_t)gridDim.x * TPB) {
        const int64_t gv = b * per + gm;
        float g[8];
        load_grad8(a, 0, (int)0, g, gv);
        if (PASS_ONLY) {
            if (a.gx) reinterpret_cast<uint4*>(a.gx)[gv] = pack8(g);
            continue;
        }
        float f[8];
        unpack8(reinterpret_cast<const uint4*>(a.x)[gv], f);
        uint32_t bc;
        const float s = flat_scale<KIND, DYN, false>(a, gv, sh, f, t, &bc);
        float gx[8];
        float part = 0.0f;
        quant_group<KIND, 8>(f, s, qmin, qmax, [&](int i, const Elem& e) {
            const float c = ste_c(e, qmin, qmax);
            gx[i] = g[i] * (e.inside ? 1.0f : 0.0f);   // g * mask (signed zero)
            part = __builtin_fmaf(g[i], c, part);
        });
        if (a.gx) reinterpret_cast<uint4*>(a.gx)[gv] = pack8(gx);
        if (a.gscale) {
            if (KIND == K_NVFP4) {
                const float tot = part + __shfl_xor(part, 1);
                if (!(gv & 1)) a.gscale[gv >> 1] = tot;
            } else {
                const float tot = group_sum(part, 1 << sh);
                if ((gv & ((1 << sh) - 1)) == 0) a.gscale[gv >> sh] = tot;
            }
        }
    }
}

// grad of a per-matrix parameter: sum of the rows' partials, fixed order
__global__ __launch_bounds__(TPB) void k_rows_to_batch(const float* rowpart, int64_t rows, float* out) {
    __shared__ float red[TPB];
    const int64_t b = blockIdx.x;
    float acc = 0.0f;
    for (int64_t r = threadIdx.x; r < rows; r += TPB) acc += rowpart[b * rows + r];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = TPB / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[b] = red[0];
}

// identity (quantiser disabled): y = x, grad_x = grad_y
__global__ __launch_bounds__(TPB) void k_copy_bf16(const uint16_t* src, int src_fp32, const void* srcv,
                                                   uint16_t* dst, int64_t nvec) {
    for (int64_t i = (int64_t)blockIdx.x * TPB + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * TPB) {
        if (src_fp32) {
            const float4* p = reinterpret_cast<const float4*>(srcv) + 2 * i;
            float4 u0 = p[0], u1 = p[1];
            float g[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            reinterpret_cast<uint4*>(dst)[i] = pack8(g);
        } else {
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
        }
    }
}

int64_t grid_flat(int64_t nvec) {
    int64_t g = (nvec + TPB - 1) / TPB;
    return g < 1 ? 1 : (g > (1 << 22) ? (1 << 22) : g);
}

int64_t grid_rows(int64_t nrows) {
    int64_t g = (nrows + RPB - 1) / RPB;
    return g < 1 ? 1 : (g > (1 << 22) ? (1 << 22) : g);
}

template <template <int, bool> class L>
hipError_t dispatch(const TensorArgs& a, hipStream_t st);

}  // namespace

size_t tensor_workspace_bytes(const QParams& q, int64_t batch, int64_t rows) {
    const bool per_tensor = (q.kind == K_NVFP4 && q.source == S_DYNAMIC) ||
                            (q.kind != K_NVFP4 && q.kind != K_NONE && q.gran == G_TENSOR &&
                             q.source == S_LEARNABLE);
    return per_tensor ? (size_t)(batch * rows) * sizeof(float) : 0;
}

#define FQ_LAUNCH(KERNEL, KIND, DYN)                                                       \
    hipLaunchKernelGGL((KERNEL<KIND, DYN>), dim3((unsigned)grid_rows(a.batch * a.rows)),   \
                       dim3(TPB), 0, st, a)
#define FQ_LAUNCH_FLAT(KERNEL, KIND, DYN)                                                  \
    hipLaunchKernelGGL((KERNEL<KIND, DYN>), dim3((unsigned)grid_flat(a.rows * (a.cols >> 3)), (unsigned)a.batch), \
                       dim3(TPB), 0, st, a)
#define FQ_KINDS(KERNEL, LAUNCH)                                                            \
    switch (a.q.kind) {                                                                     \
    case K_NVFP4: if (dyn) LAUNCH(KERNEL, K_NVFP4, true); else LAUNCH(KERNEL, K_NVFP4, false); break; \
    case K_INT: if (dyn) LAUNCH(KERNEL, K_INT, true); else LAUNCH(KERNEL, K_INT, false); break;       \
    default: if (dyn) LAUNCH(KERNEL, K_FP8, true); else LAUNCH(KERNEL, K_FP8, false); break;          \
    }

#define FQ_LAUNCH_C(KERNEL, KIND, DYN)                                                     \
    do {                                                                                   \
        if (codes) FQ_LAUNCH_GRID(KERNEL, KIND, DYN, true);                                \
        else FQ_LAUNCH_GRID(KERNEL, KIND, DYN, false);                                     \
    } while (0)

hipError_t launch_tensor_fwd(const TensorArgs& a, hipStream_t st) {
    const int64_t nrows = a.batch * a.rows;
    if (nrows == 0 || a.cols == 0) return hipSuccess;
    const bool dyn = a.q.source == S_DYNAMIC;
    const bool codes = a.codes || a.bcodes;
    switch (a.q.kind) {
    case K_NONE: {
        if (!a.y || a.y == a.x) return hipSuccess;
        const int64_t nvec = nrows * a.cols / 8;
        hipLaunchKernelGGL(k_copy_bf16, dim3((unsigned)grid_rows(nvec / 16 + 1)), dim3(TPB), 0, st,
                           a.x, 0, nullptr, a.y, nvec);
        break;
    }
    case K_NVFP4:
    case K_INT:
    case K_FP8:
        // NVFP4 blocks and groups flat; per-row / per-tensor scales a row per wave
        if ((a.q.kind == K_NVFP4 || a.q.gran == G_GROUP) && a.batch <= 65535) {
#define FQ_LAUNCH_GRID(KERNEL, KIND, DYN, C)                                                \
    hipLaunchKernelGGL((KERNEL<KIND, DYN, C>), dim3((unsigned)grid_flat(a.rows * (a.cols >> 3)), (unsigned)a.batch), \
                       dim3(TPB), 0, st, a)
            FQ_KINDS(k_tensor_fwd_flat, FQ_LAUNCH_C)
#undef FQ_LAUNCH_GRID
        } else {
#define FQ_LAUNCH_GRID(KERNEL, KIND, DYN, C)                                                \
    hipLaunchKernelGGL((KERNEL<KIND, DYN, C>), dim3((unsigned)grid_rows(a.batch * a.rows)), dim3(TPB), 0, st, a)
            FQ_KINDS(k_tensor_fwd, FQ_LAUNCH_C)
#undef FQ_LAUNCH_GRID
        }
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_tensor_bwd(const TensorArgs& a, hipStream_t st) {
    const int64_t nrows = a.batch * a.rows;
    if (nrows == 0 || a.cols == 0) return hipSuccess;
    const bool dyn = a.q.source == S_DYNAMIC;
    switch (a.q.kind) {
    case K_NONE: {
        if (!a.gx) return hipSuccess;
        const int64_t nvec = nrows * a.cols / 8;
        hipLaunchKernelGGL(k_copy_bf16, dim3((unsigned)grid_rows(nvec / 16 + 1)), dim3(TPB), 0, st,
                           static_cast<const uint16_t*>(a.gy), a.gy_fp32, a.gy, a.gx, nvec);
        return hipGetLastError();
    }
    case K_NVFP4:
    case K_INT:
    case K_FP8: {
        // row reductions (per-row / per-tensor gradients, the NVFP4 tensor
        // scale of dynamic blocks) need a row per wave; else flat
        const bool flat = (a.q.kind == K_NVFP4 ? !dyn : (dyn || a.q.gran == G_GROUP)) && a.batch <= 65535;
        if (flat) { FQ_KINDS(k_tensor_bwd_flat, FQ_LAUNCH_FLAT) }
        else { FQ_KINDS(k_tensor_bwd, FQ_LAUNCH) }
        break;
    }
    default: return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.gscale && tensor_workspace_bytes(a.q, a.batch, a.rows) > 0) {
        hipLaunchKernelGGL(k_rows_to_batch, dim3((unsigned)a.batch), dim3(TPB), 0, st,
                           a.rowpart, a.rows, a.gscale);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace fq
