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

// Two fp32 -> packed bf16 pair (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 with both operands (two scalar casts become two
// conversions, a shift and an or).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                      pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
}

// ------------------------------------------------------------ scalar loads --
// p[i] through the scalar cache when i is wave-uniform, for an array the
// kernel does not write.  (A plain load in a kernel that also stores is a
// vector load, and a wait for it waits for every vector memory operation
// issued before it, stores included.)
__device__ __forceinline__ int32_t sload(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
__device__ __forceinline__ float sload(const float* p, int64_t i) {
    return ((const __attribute__((address_space(4))) float*)p)[i];
}

// s_waitcnt vmcnt(N) through the builtin, so that the compiler's own wait
// bookkeeping sees it (the loads it tracks that are older than the N most
// recent count as complete, as they are), then a compiler barrier, so that
// no memory access moves across the wait.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);   // expcnt, lgkmcnt: no wait
    asm volatile("" ::: "memory");
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
// Round to nearest, ties to even, onto the E4M3FN and E2M1 grids with the
// gfx950 conversion instructions (v_cvt_pk_fp8_f32 / v_cvt_f32_fp8 and
// v_cvt_scalef32_pk_fp4_f32 / v_cvt_scalef32_pk_f32_fp4 with scale 1).  On the
// box they agree bit for bit with the closed-form rounding (E4M3: subnormal
// spacing 2^-9 below 2^-6, three mantissa bits above; E2M1: spacing 0.5 below
// 2, 1 in [2, 4), 2 in [4, 6]) for every fp32 magnitude up to the largest
// grid value, subnormals and ties included.  Callers saturate first.
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));

// E4M3FN value of a magnitude in [0, 448]; *code gets the 7-bit magnitude code.
__device__ __forceinline__ float e4m3_round(float a, uint32_t* code) {
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, a, 0, false);
    *code = (uint32_t)p & 0x7Fu;
    return __builtin_amdgcn_cvt_f32_fp8(p, 0);
}
__device__ __forceinline__ float e4m3_round(float a) {
    return __builtin_amdgcn_cvt_f32_fp8(__builtin_amdgcn_cvt_pk_fp8_f32(a, a, 0, false), 0);
}
// two at once (one conversion each way for the pair)
__device__ __forceinline__ void e4m3_round2(float a0, float a1, float* q0, float* q1) {
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    *q0 = __builtin_amdgcn_cvt_f32_fp8(p, 0);
    *q1 = __builtin_amdgcn_cvt_f32_fp8(p, 1);
}

// E2M1 value of a magnitude in [0, 6]; ties go to the even code.
__device__ __forceinline__ float e2m1_round(float a) {
    const unsigned p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, a, 1.0f, 0);
    const f32x2_cvt b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    return b.x;
}
__device__ __forceinline__ void e2m1_round2(float a0, float a1, float* q0, float* q1) {
    const unsigned p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a0, a1, 1.0f, 0);
    const f32x2_cvt b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    *q0 = b.x;
    *q1 = b.y;
}
// E2M1 grid values (RNE) of eight quotients: the four pairs go into the four
// bytes of one packed word and back.  The conversion saturates: beyond +-6,
// infinities and NaN give +-6 with the operand's sign bit (measured on
// gfx950), so it needs no clamp; a caller that must take the sign from
// elsewhere (a NaN's sign after arithmetic is not defined) copies it after.
__device__ __forceinline__ void e2m1_round8(const float* r, float* q) {
    unsigned p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r[0], r[1], 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, r[2], r[3], 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, r[4], r[5], 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, r[6], r[7], 1.0f, 3);
    const f32x2_cvt b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    const f32x2_cvt b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1);
    const f32x2_cvt b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2);
    const f32x2_cvt b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3);
    q[0] = b0.x; q[1] = b0.y; q[2] = b1.x; q[3] = b1.y;
    q[4] = b2.x; q[5] = b2.y; q[6] = b3.x; q[7] = b3.y;
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
// 1/d correctly rounded for d in [2^-120, 2^120]: one Newton step with FMAs
// from the hardware reciprocal (within an ulp); on gfx950 this equals the IEEE
// reciprocal for every significand at every exponent of that range.
__device__ __forceinline__ float rcp_rn(float d) {
    const float y0 = __builtin_amdgcn_rcpf(d);
    return __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
}

struct Div {
    float s, inv;      // inv: RN(1/s), meaningful (and used) only when fast
    bool fast;
    __device__ __forceinline__ void set(float s_) {
        s = s_;
        fast = (s_ >= 0x1p-120f) && (s_ <= 0x1p120f);
        inv = rcp_rn(s_);
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
// no zero case and the corrected division only, so no branches; the grid
// value is left to the caller
template <int KIND>
__device__ __forceinline__ Elem quant_fast_r(float x, const Div& d, float qmin, float qmax) {
    const float q0 = x * d.inv;
    const float rem = __builtin_fmaf(-q0, d.s, x);
    const float r = __builtin_fmaf(rem, d.inv, q0);
    Elem e;
    e.r = r;
    // NVFP4 and FP8 grids are symmetric (qmin = -qmax)
    e.inside = KIND == K_INT ? (r >= qmin) && (r <= qmax) : fabsf(r) <= qmax;
    return e;
}

// grid values of two divided elements (signs from x), one conversion pair
template <int KIND>
__device__ __forceinline__ void grid_q2(Elem& e0, Elem& e1, float x0, float x1, float qmin, float qmax) {
    if (KIND == K_NVFP4) {
        float q0, q1;
        e2m1_round2(fminf(fabsf(e0.r), 6.0f), fminf(fabsf(e1.r), 6.0f), &q0, &q1);
        e0.q = copysignf(q0, x0);
        e1.q = copysignf(q1, x1);
    } else if (KIND == K_FP8) {
        float q0, q1;
        e4m3_round2(fminf(fabsf(e0.r), 448.0f), fminf(fabsf(e1.r), 448.0f), &q0, &q1);
        e0.q = copysignf(q0, x0);
        e1.q = copysignf(q1, x1);
    } else {
        e0.q = grid_q<KIND>(e0.r, x0, qmin, qmax);
        e1.q = grid_q<KIND>(e1.r, x1, qmin, qmax);
    }
}

// Run f(i, Elem) over the N elements x[0..N) sharing the effective scale s.
// The wave takes the branch-free path when every active lane's scale is in
// the normal range (a wave-uniform branch), else the general one.
template <int KIND, int N, typename F>
__device__ __forceinline__ void quant_group(const float* x, float s, float qmin, float qmax, F&& f) {
    static_assert(N % 2 == 0, "elements come in pairs");
    Div dv;
    dv.set(s);
    if (__all(dv.fast)) {
        Elem e[N];
#pragma unroll
        for (int i = 0; i < N; ++i) e[i] = quant_fast_r<KIND>(x[i], dv, qmin, qmax);
        if constexpr (KIND == K_NVFP4 && N % 8 == 0) {
            // saturating conversion of the signed quotients, sign from x: the
            // same values as copysign(e2m1(min(|r|, 6)), x) for every r
#pragma unroll
            for (int i = 0; i < N; i += 8) {
                float rr[8], qq[8];
#pragma unroll
                for (int v = 0; v < 8; ++v) rr[v] = e[i + v].r;
                e2m1_round8(rr, qq);
#pragma unroll
                for (int v = 0; v < 8; ++v) e[i + v].q = copysignf(qq[v], x[i + v]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < N; i += 2) grid_q2<KIND>(e[i], e[i + 1], x[i], x[i + 1], qmin, qmax);
        }
#pragma unroll
        for (int i = 0; i < N; ++i) f(i, e[i]);
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
