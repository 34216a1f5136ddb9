// Single-token decode step for gfx950: the recurrent mode of the selective
// SSM, which keeps a fixed-size state per channel and advances it one token
// at a time ("Mamba架构深度剖析：如何以线性时间重塑序列建模" §3).  For each
// (b, d):  Δ = softplus(dt + dt_bias),  h_n <- exp(Δ A_n) h_n + B̄_n x with the
// zero-order-hold B̄_n = expm1(Δ A_n)/A_n B_n (Δ B_n at A_n = 0)
// ("Mamba架构与SSM模型：高效序列建模技术解析" §2.1-2.2), then
// y = (sum_n C_n h_n + D x) * SiLU(z).
// HBM-bound: the fp32 state (N*4 bytes read and written per channel) dominates
// the traffic, so one lane owns one channel, reads its state row with 128-bit
// loads when N = 16, and B/C of the batch row are wave-uniform scalar loads.
#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

constexpr int kThreads = 256;

template <bool BF16>
__global__ void __launch_bounds__(kThreads) state_update_kernel(
    float *__restrict__ h, const void *__restrict__ x_, const void *__restrict__ dt_,
    const float *__restrict__ dt_bias, const float *__restrict__ A, const void *__restrict__ Bm_,
    const void *__restrict__ Cm_, const float *__restrict__ Dskip, const void *__restrict__ z_,
    void *__restrict__ y_, int64_t D, int N, int vec16, int64_t blocks_per_row)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    const int64_t b = (int64_t)blockIdx.x / blocks_per_row;
    const int64_t d = ((int64_t)blockIdx.x - b * blocks_per_row) * kThreads + threadIdx.x;
    if (d >= D)
        return;
    const int64_t c = b * D + d;
    float hs[kMaxN], Ar[kMaxN], Bv[kMaxN], Cv[kMaxN];
    const T *Bm = reinterpret_cast<const T *>(Bm_) + b * N;
    const T *Cm = reinterpret_cast<const T *>(Cm_) + b * N;
    if (vec16) {
        const float4 *hq = reinterpret_cast<const float4 *>(h + c * kMaxN);
        const float4 *aq = reinterpret_cast<const float4 *>(A + d * kMaxN);
#pragma unroll
        for (int i = 0; i < kMaxN / 4; ++i) {
            const float4 hv = hq[i], av = aq[i];
            hs[4 * i] = hv.x; hs[4 * i + 1] = hv.y; hs[4 * i + 2] = hv.z; hs[4 * i + 3] = hv.w;
            Ar[4 * i] = av.x; Ar[4 * i + 1] = av.y; Ar[4 * i + 2] = av.z; Ar[4 * i + 3] = av.w;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kMaxN; ++n) {
            hs[n] = (n < N) ? h[c * N + n] : 0.f;
            Ar[n] = (n < N) ? A[d * N + n] : 0.f;
        }
    }
#pragma unroll
    for (int n = 0; n < kMaxN; ++n) {
        Bv[n] = (n < N) ? E::load(Bm + n) : 0.f;
        Cv[n] = (n < N) ? E::load(Cm + n) : 0.f;
    }
    const float xv = E::load(reinterpret_cast<const T *>(x_) + c);
    const float dtv = E::load(reinterpret_cast<const T *>(dt_) + c);
    const float bias = dt_bias ? dt_bias[d] : 0.f;
    const float l = softplus_log2(fmaf(dtv, kLog2e, bias * kLog2e));  // Δ / ln 2
    const float delta = l * kLn2;
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < kMaxN; ++n) {
        const float an = Ar[n];
        const float en = (an == 0.f) ? 1.f : hw_exp2(an * l);
        const float coef = (an == 0.f) ? delta : expm1f(an * delta) / an;
        hs[n] = fmaf(en, hs[n], coef * (Bv[n] * xv));
        acc = fmaf(Cv[n], hs[n], acc);
    }
    float yv = acc + (Dskip ? Dskip[d] : 0.f) * xv;
    if (z_)
        yv *= silu_hw(E::load(reinterpret_cast<const T *>(z_) + c));
    E::store(reinterpret_cast<T *>(y_) + c, yv);
    if (vec16) {
        float4 *hq = reinterpret_cast<float4 *>(h + c * kMaxN);
#pragma unroll
        for (int i = 0; i < kMaxN / 4; ++i)
            hq[i] = make_float4(hs[4 * i], hs[4 * i + 1], hs[4 * i + 2], hs[4 * i + 3]);
    } else {
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            if (n < N)
                h[c * N + n] = hs[n];
    }
}

}  // namespace

hipError_t launch_state_update(const StepArgs &a, hipStream_t s)
{
    if (a.B * a.D == 0)
        return hipSuccess;
    const int vec16 = (a.N == kMaxN && ((uintptr_t)a.h % 16) == 0 && ((uintptr_t)a.A % 16) == 0);
    const int64_t bpr = (a.D + kThreads - 1) / kThreads;
    dim3 grid((unsigned)(bpr * a.B));
    if (a.bf16)
        hipLaunchKernelGGL(state_update_kernel<true>, grid, dim3(kThreads), 0, s, a.h, a.x, a.dt,
                           a.dt_bias, a.A, a.Bm, a.Cm, a.Dskip, a.z, a.y, a.D, a.N, vec16, bpr);
    else
        hipLaunchKernelGGL(state_update_kernel<false>, grid, dim3(kThreads), 0, s, a.h, a.x,
                           a.dt, a.dt_bias, a.A, a.Bm, a.Cm, a.Dskip, a.z, a.y, a.D, a.N, vec16, bpr);
    return hipGetLastError();
}

}  // namespace mamba
