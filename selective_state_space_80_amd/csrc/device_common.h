// Device-side helpers shared by the kernels: element conversion and the
// hardware transcendental instructions of gfx950 (v_exp_f32 = 2^x,
// v_log_f32 = log2 x, v_rcp_f32 = 1/x).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mamba {

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// two floats -> a packed bf16 pair (a in the low half), round to nearest even
// (one v_cvt_pk_bf16_f32); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return cvt2(f, 0.f) & 0xffffu; }

// Element load / store for the two I/O types.
template <bool BF16> struct Elem;
template <> struct Elem<false> {
    using T = float;
    static __device__ __forceinline__ float load(const T *p) { return *p; }
    static __device__ __forceinline__ void store(T *p, float v) { *p = v; }
};
template <> struct Elem<true> {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T *p) { return bf16_bits_to_f32(*p); }
    static __device__ __forceinline__ void store(T *p, float v) {
        *p = (uint16_t)f32_to_bf16_bits(v);
    }
};

// z * sigmoid(z) with the hardware exp2 / rcp.
__device__ __forceinline__ float silu_hw(float z) {
    return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

// softplus(v) in log2 units: log2(1 + t), t = 2^v2, for v2 = v * log2(e).
// Above v2 = 25 the 1 no longer changes 1 + t in fp32, so the value is v2
// itself; taking it directly also keeps t from overflowing to +inf for
// v2 >= 128.  Below v2 = -6 (t < 1/64) the value is small and
// v_log_f32(1 + t) would carry its error near 1, an absolute one, which is a
// large relative error in a small Δ (1.6e-3 in the outputs of a scan with Δ
// near 1e-5): there it is the series log2(e) (t - t^2/2 + t^3/3), whose
// truncation stays below 6e-7 relative.
__device__ __forceinline__ float softplus_log2(float v2) {
    const float t = hw_exp2(v2);
    const float l = hw_log2(1.0f + t);
    constexpr float c1 = 1.44269504088896341f, c2 = -c1 / 2.f, c3 = c1 / 3.f;
    const float small = t * fmaf(fmaf(c3, t, c2), t, c1);
    return v2 > 25.0f ? v2 : (v2 < -6.0f ? small : l);
}

// Input coefficient of the exact ZOH step for one state, B̄_n / B_n =
// (exp(ΔA_n) - 1) / A_n = Δ φ1(ΔA_n) with φ1(v) = (e^v - 1)/v, given
// en = exp(ΔA_n).  For |ΔA_n| < 1/8, φ1 by its Taylor series through v^4
// (truncation below 5e-8 relative; A_n = 0 gives exactly Δ, the limit);
// otherwise (en - 1)/A_n, where |en - 1| > 0.117 keeps the subtraction's
// relative error near 1e-6.
__device__ __forceinline__ float zoh_input_coef(float an, float delta, float en)
{
    const float v = an * delta;
    float phi = 1.f / 120.f;  // 1/5!
    phi = fmaf(phi, v, 1.f / 24.f);
    phi = fmaf(phi, v, 1.f / 6.f);
    phi = fmaf(phi, v, 0.5f);
    phi = fmaf(phi, v, 1.f);
    return fabsf(v) < 0.125f ? delta * phi : (en - 1.f) * hw_rcp(an);
}

// The same coefficient taken from w = ΔA_n log2(e), the exponent already formed
// for en = 2^w, with 1/A_n supplied:  for |ΔA_n| < 1/8 the series of φ1 through
// v^4 written in w (coefficients ln2^k/(k+1)!; truncation below 5e-8
// relative), otherwise (en - 1)/A_n.
__device__ __forceinline__ float zoh_coef_w(float w, float delta, float en, float rcpa)
{
    constexpr float c1 = 0.693147180559945309f;  // ln 2
    constexpr float c2 = c1 * c1, c3 = c2 * c1, c4 = c3 * c1;
    float phi = c4 / 120.f;
    phi = fmaf(phi, w, c3 / 24.f);
    phi = fmaf(phi, w, c2 / 6.f);
    phi = fmaf(phi, w, c1 / 2.f);
    phi = fmaf(phi, w, 1.f);
    return fabsf(w) < 0.125f * 1.44269504088896341f ? delta * phi : (en - 1.f) * rcpa;
}

// Sum over the four lanes of a quad, the result in all four: two DPP quad
// permutes (lane ^ 1, then lane ^ 2), no LDS traffic.
__device__ __forceinline__ float quad_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    return v;
}

}  // namespace mamba
