// Device helpers shared by the fake-quant kernels (gfx950, wave64).
//
// Numbers of one quantiser (AngelSlim "MCoreQAD Backend" page: weights frozen,
// fake quantisation, only scales trained; nxmr.cn article section 二.3):
//   r = x / s^ correctly rounded, q = nearest grid value of clamp(r) (ties to
//   the even code), y = bf16_rne(q * s^); straight-through backward
//   c = q - r inside [qmin, qmax], the bound outside.
// Every step below is a single IEEE fp32 operation; the library is compiled with
// -ffp-contract=off so nothing is fused behind our back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

constexpr int WAVE = 64;

enum Kind : int { K_NONE = 0, K_NVFP4 = 1, K_INT = 2, K_FP8 = 3 };
enum Gran : int { G_TENSOR = 0, G_ROW = 1, G_GROUP = 2 };
enum Source : int { S_LEARNABLE = 0, S_STATIC = 1, S_DYNAMIC = 2 };

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    __bf16 ha = (__bf16)a, hb = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                      pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
}

// ------------------------------------------------------------- reductions ---
// Fixed xor-butterfly trees: the same order on every call, so sums are
// bitwise reproducible.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < WAVE; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < WAVE; m <<= 1) v = v + __shfl_xor(v, m);
    return v;
}
// reduce over aligned groups of `lanes` lanes (power of two <= 64)
__device__ __forceinline__ float group_max(float v, int lanes) {
    for (int m = 1; m < lanes; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float group_sum(float v, int lanes) {
    for (int m = 1; m < lanes; m <<= 1) v = v + __shfl_xor(v, m);
    return v;
}

// ----------------------------------------------------------------- grids ---
// E4M3FN round-to-nearest-even of a magnitude in [0, 448] (callers saturate
// first).  Returns the value; *code gets the 7-bit magnitude code.  Both the
// subnormal (spacing 2^-9 below 2^-6) and the normal rounding are formed and
// one is selected, so lanes never diverge.
__device__ __forceinline__ float e4m3_round(float a, uint32_t* code) {
    const float m = rintf(a * 512.0f);                 // exact scaling, ties to even
    uint32_t u = __float_as_uint(a);
    u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;   // keep 3 mantissa bits
    const bool sub = a < 0.015625f;
    *code = sub ? (uint32_t)m : ((((u >> 23) - 120u) << 3) | ((u >> 20) & 7u));   // 8 == 2^-6, code 0x08
    return sub ? m * 0.001953125f : __uint_as_float(u);
}
__device__ __forceinline__ float e4m3_round(float a) {
    const float m = rintf(a * 512.0f);
    uint32_t u = __float_as_uint(a);
    u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
    return a < 0.015625f ? m * 0.001953125f : __uint_as_float(u);
}

// E2M1 round-to-nearest-even of a magnitude in [0, 6]: spacing 0.5 below 2,
// 1 in [2, 4), 2 in [4, 6]; rint breaks ties to the even multiple, which is
// the even code.
// Computed as (a + C) - C with C = 2^22, 2^23, 2^24 for spacing 0.5, 1, 2:
// the fp32 sum rounds a to a multiple of ulp(C), ties to the even multiple;
// C = 2^(21 + clamp(exponent of a, 1, 3)) with a = m 2^e, m in [0.5, 1).
__device__ __forceinline__ float e2m1_round(float a) {
    const int e = __builtin_amdgcn_frexp_expf(a);
    const float c = __uint_as_float((uint32_t)(min(max(e, 1), 3) + 148) << 23);   // 2^(21 + e)
    return (a + c) - c;
}
// 3-bit magnitude code of an E2M1 grid value: from 1 up, exponent and top
// mantissa bit of the fp32 pattern; below 1 (0 or 0.5), 2 qm read off the low
// bits of 2 qm + 2^23.  Both formed, one selected: no divergent branch.
__device__ __forceinline__ uint32_t e2m1_code(float qm) {
    const uint32_t hi = (__float_as_uint(qm) >> 22) - 252u;
    const uint32_t lo = __float_as_uint(qm * 2.0f + 8388608.0f) & 1u;
    return qm >= 1.0f ? hi : lo;
}

// --------------------------------------------------------------- division ---
// r = x / s correctly rounded, given inv = 1/s correctly rounded and s in the
// normal range [2^-120, 2^120] (Markstein's correction step: q0 = x*inv, the
// exact remainder x - q0*s by FMA, one corrected rounding).
struct Div {
    float s, inv;
    bool fast;
    __device__ __forceinline__ void set(float s_) {
        s = s_;
        inv = 1.0f / s_;
        fast = (s_ >= 0x1p-120f) && (s_ <= 0x1p120f);
    }
    __device__ __forceinline__ float operator()(float x) const {
        if (fast) {
            float q0 = x * inv;
            float rem = __builtin_fmaf(-q0, s, x);
            return __builtin_fmaf(rem, inv, q0);
        }
        return x / s;
    }
};

// One element through the quantiser.  Returns q (signed grid value, sign of
// x); r and `inside` for the backward.  s == 0 gives q = +-0, r = +-0, inside.
struct Elem {
    float q, r;
    bool inside;
};

// grid value of r (sign of x), r already divided
template <int KIND>
__device__ __forceinline__ float grid_q(float r, float x, float qmin, float qmax) {
    if (KIND == K_INT) return copysignf(rintf(fminf(fmaxf(r, qmin), qmax)), x);   // sign from x:
    if (KIND == K_NVFP4) return copysignf(e2m1_round(fminf(fabsf(r), 6.0f)), x);    // the corrected
    return copysignf(e4m3_round(fminf(fabsf(r), 448.0f)), x);                        // division gives +0 for -0
}

template <int KIND>
__device__ __forceinline__ Elem quant_elem(float x, const Div& d, float qmin, float qmax) {
    Elem e;
    if (d.s == 0.0f) {
        e.q = copysignf(0.0f, x);
        e.r = e.q;
        e.inside = true;
        return e;
    }
    const float r = d(x);
    e.r = r;
    e.inside = (r >= qmin) && (r <= qmax);
    e.q = grid_q<KIND>(r, x, qmin, qmax);
    return e;
}

// quant_elem for a scale known to be in the normal range [2^-120, 2^120]:
// no zero case and the corrected division only, so no branches
template <int KIND>
__device__ __forceinline__ Elem quant_fast(float x, const Div& d, float qmin, float qmax) {
    const float q0 = x * d.inv;
    const float rem = __builtin_fmaf(-q0, d.s, x);
    const float r = __builtin_fmaf(rem, d.inv, q0);
    Elem e;
    e.r = r;
    // NVFP4 and FP8 grids are symmetric (qmin = -qmax)
    e.inside = KIND == K_INT ? (r >= qmin) && (r <= qmax) : fabsf(r) <= qmax;
    e.q = grid_q<KIND>(r, x, qmin, qmax);
    return e;
}

// Run f(i, Elem) over the N elements x[0..N) sharing the effective scale s.
// The wave takes the branch-free path when every active lane's scale is in
// the normal range (a wave-uniform branch), else the general one.
template <int KIND, int N, typename F>
__device__ __forceinline__ void quant_group(const float* x, float s, float qmin, float qmax, F&& f) {
    Div dv;
    dv.set(s);
    if (__all(dv.fast)) {
#pragma unroll
        for (int i = 0; i < N; ++i) f(i, quant_fast<KIND>(x[i], dv, qmin, qmax));
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) f(i, quant_elem<KIND>(x[i], dv, qmin, qmax));
    }
}

// c = d y / d s^ (straight-through): q - r inside, the bound outside.  Outside
// the range q is the clamped grid value, which is that bound (the bounds lie
// on the grid and q takes the sign of r), so c = q - (inside ? r : 0) with no
// branch.
__device__ __forceinline__ float ste_c(const Elem& e, float qmin, float qmax) {
    (void)qmin;
    (void)qmax;
    return e.q - (e.inside ? e.r : 0.0f);
}

// code of one element (4-bit value in the low bits, or 8-bit)
template <int KIND>
__device__ __forceinline__ uint32_t elem_code(const Elem& e, float x) {
    uint32_t sgn = __float_as_uint(x) >> 31;
    if (KIND == K_NVFP4) return (sgn << 3) | e2m1_code(fabsf(e.q));
    if (KIND == K_FP8) {
        uint32_t c;
        e4m3_round(fabsf(e.q), &c);            // exact: q is already on the grid
        return (sgn << 7) | c;
    }
    return (uint32_t)(int32_t)e.q & 0xFFu;     // two's complement; INT4 keeps the low nibble
}

}  // namespace fq
