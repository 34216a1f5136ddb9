// Single-token decode step for gfx950: the recurrent mode of the selective
// SSM, which keeps a fixed-size state per channel and advances it one token
// at a time ("Mamba架构深度剖析：如何以线性时间重塑序列建模" §3).  For each
// (b, d):  Δ = softplus(dt + dt_bias),  h_n <- exp(Δ A_n) h_n + B̄_n x with the
// zero-order-hold B̄_n = (exp(Δ A_n) - 1)/A_n B_n (Δ B_n at A_n = 0)
// ("Mamba架构与SSM模型：高效序列建模技术解析" §2), then
// y = (sum_n C_n h_n + D x) * SiLU(z).
// Bound by memory: the fp32 state (N*4 bytes read and written per channel)
// dominates the traffic.  NT: the state is loaded and stored with nontemporal
// hints, for callers whose state leaves the caches between two steps anyway
// (a model's layers each touch their own state once per token).  With N = 16 and aligned rows, four lanes share a
// channel, one 16-byte quarter of its state each, so every load and store of
// a wave covers one contiguous 1 KB run; the readout is summed over the four
// lanes with two DPP quad permutes.  Other N: one lane per channel.
// With the conv front end fused in front (KC taps), x is the raw input: the
// step's scan input is SiLU(conv_b + sum_k conv_w[d,k] u_k) over the KC - 1
// carried raw inputs and the new one, and the window moves by one slot
// ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式" §3.1).
#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

constexpr int kThreads = 256;
// channel quads per lane: two, 64 quads apart, keep twice the bytes in flight
// per lane (one measured 2-6% slower, four slower still: fewer waves fit)
constexpr int kQuadsPerLane = 2;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Quarter i4 of the state (16 bytes), plain or nontemporal.
template <bool NT>
__device__ __forceinline__ void load_state4(const float *h, int64_t i4, float (&v)[4])
{
    const f32x4 *p = reinterpret_cast<const f32x4 *>(h) + i4;
    f32x4 t;
    if constexpr (NT)
        t = __builtin_nontemporal_load(p);
    else
        t = *p;
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
}

template <bool NT>
__device__ __forceinline__ void store_state4(float *h, int64_t i4, const float (&v)[4])
{
    const f32x4 t = {v[0], v[1], v[2], v[3]};
    f32x4 *p = reinterpret_cast<f32x4 *>(h) + i4;
    if constexpr (NT)
        __builtin_nontemporal_store(t, p);
    else
        *p = t;
}

template <bool NT>
__device__ __forceinline__ float load_state(const float *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT>
__device__ __forceinline__ void store_state(float *p, float v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <bool BF16>
__device__ __forceinline__ void load4(const void *base, int64_t i4, float (&v)[4])
{
    if constexpr (BF16) {
        const uint2 w = reinterpret_cast<const uint2 *>(base)[i4];
        v[0] = __uint_as_float(w.x << 16);
        v[1] = __uint_as_float(w.x & 0xffff0000u);
        v[2] = __uint_as_float(w.y << 16);
        v[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
        const float4 f = reinterpret_cast<const float4 *>(base)[i4];
        v[0] = f.x;
        v[1] = f.y;
        v[2] = f.z;
        v[3] = f.w;
    }
}

// The conv front end of one channel (flat index c, channel d), KC >= 1 taps:
// its inputs (the KC - 1 carried raw inputs, then x_raw), weights and bias.
template <bool BF16, int KC>
struct ConvStep {
    float u[KC], w[KC], b;
    __device__ __forceinline__ void load(const void *state, float x_raw, const float *conv_w,
                                         const float *bias_p, int64_t c, int64_t d)
    {
        using E = Elem<BF16>;
        const typename E::T *st = reinterpret_cast<const typename E::T *>(state) + c * (KC - 1);
#pragma unroll
        for (int k = 0; k < KC - 1; ++k)
            u[k] = E::load(st + k);
        u[KC - 1] = x_raw;
#pragma unroll
        for (int k = 0; k < KC; ++k)
            w[k] = conv_w[d * KC + k];
        b = bias_p[d];
    }
    __device__ __forceinline__ float out(float bias_on) const
    {
        float acc = bias_on * b;
#pragma unroll
        for (int k = 0; k < KC; ++k)
            acc = fmaf(w[k], u[k], acc);
        return silu_hw(acc);
    }
    // slot j (< KC - 1, a constant after unrolling) of the window after this step
    __device__ __forceinline__ void store_slot(void *state, int64_t c, int j) const
    {
        using E = Elem<BF16>;
        E::store(reinterpret_cast<typename E::T *>(state) + c * (KC - 1) + j, u[j + 1]);
    }
};

// N = 16, state and A rows 16-byte aligned, B/C rows aligned to 4 elements.
// Grid: x over one batch row's 4 D quads, y over batch rows from b0 (the host
// launches once per 65535 rows).  A wave handles QPT runs of 64 quads (16 channels each): lane l
// of wave w takes row quads w*64*QPT + k*64 + l, k < QPT, i.e. states
// [4q, 4q+4), q = l % 4, of QPT channels, so each of its loads and stores
// covers one contiguous 1 KB run per wave while QPT of them are in flight per
// lane.  Every load of a lane is issued before the first use (no branch
// between them: an absent dt_bias, Dskip or z is read through another valid
// pointer and its value ignored).
// KC > 0: the conv front end first.  Lane q of a quad holds tap q (window
// slot q, or the raw input for the last tap; lanes past the taps weigh 0):
// one 2-byte and one 4-byte load per lane, the weighted taps summed over the
// quad like the readout, and lane q in 1..KC-1 writes its tap to slot q - 1.
template <bool BF16, int QPT, int KC, bool NT>
__global__ void __launch_bounds__(kThreads) state_update_quad_kernel(
    float *__restrict__ h, const void *__restrict__ x_, const void *__restrict__ dt_,
    const float *__restrict__ dt_bias, const float *__restrict__ A, const void *__restrict__ Bm_,
    const void *__restrict__ Cm_, const float *__restrict__ Dskip, const void *__restrict__ z_,
    void *__restrict__ y_, int64_t b0, int64_t D, void *__restrict__ conv_state,
    const float *__restrict__ conv_w, const float *__restrict__ conv_b)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    const int64_t b = b0 + blockIdx.y;
    const int lane = (int)(threadIdx.x & 63);
    const int q = lane & 3;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t row_quads = 4 * D;
    const float *bias_p = dt_bias ? dt_bias : A;  // A has at least D entries
    const float bias_on = dt_bias ? 1.f : 0.f;
    const float *skip_p = Dskip ? Dskip : A;
    const float skip_on = Dskip ? 1.f : 0.f;
    const T *z_p = reinterpret_cast<const T *>(z_ ? z_ : x_);  // same shape as x
    const float *cb_p = conv_b ? conv_b : conv_w;  // conv_w has at least D entries
    const float cb_on = conv_b ? 1.f : 0.f;
    {
        float hs[QPT][4], a[QPT][4], Bv[4], Cv[4], xv[QPT], dtv[QPT], bias[QPT], zv[QPT], dsk[QPT];
        float tu[QPT], tw[QPT], tb[QPT];  // this lane's conv tap: input, weight; conv bias
        const int tap = KC > 0 ? (q < KC ? q : KC - 1) : 0;
        const float tap_on = q < KC ? 1.f : 0.f;
        int64_t gq[QPT], cq[QPT], dq[QPT];
        bool live[QPT];
        load4<BF16>(Bm_, b * 4 + q, Bv);
        load4<BF16>(Cm_, b * 4 + q, Cv);
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int64_t rq = (wave * QPT + k) * 64 + lane;  // quad within the row
            // whole channels per run of 64 quads, so a lane past the end only
            // ever shares its quad sums with lanes past the end too
            live[k] = rq < row_quads;
            const int64_t rqc = live[k] ? rq : row_quads - 1;
            dq[k] = rqc >> 2;
            cq[k] = b * D + dq[k];
            gq[k] = b * row_quads + rqc;
            load_state4<NT>(h, gq[k], hs[k]);
            load4<false>(A, dq[k] * 4 + q, a[k]);
            xv[k] = E::load(reinterpret_cast<const T *>(x_) + cq[k]);
            dtv[k] = E::load(reinterpret_cast<const T *>(dt_) + cq[k]);
            bias[k] = bias_p[dq[k]];
            zv[k] = E::load(z_p + cq[k]);
            dsk[k] = skip_p[dq[k]];
            if constexpr (KC > 0) {
                tu[k] = xv[k];
                if constexpr (KC > 1) {
                    const T *win = reinterpret_cast<const T *>(conv_state) + cq[k] * (KC - 1);
                    const float u = E::load(win + (tap < KC - 1 ? tap : KC - 2));
                    tu[k] = tap < KC - 1 ? u : xv[k];
                }
                tw[k] = conv_w[dq[k] * KC + tap];
                tb[k] = cb_p[dq[k]];
            }
        }
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            if constexpr (KC > 0) {  // the scan input of this step
                float part = tap_on * tw[k] * tu[k];
                xv[k] = silu_hw(quad_sum(part) + cb_on * tb[k]);
            }
            const float l =
                softplus_log2(fmaf(dtv[k], kLog2e, bias_on * bias[k] * kLog2e));  // Δ / ln 2
            const float delta = l * kLn2;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float en = hw_exp2(a[k][i] * l);  // exp(Δ A_n); 1 when A_n = 0
                const float coef = zoh_input_coef(a[k][i], delta, en);
                hs[k][i] = fmaf(en, hs[k][i], coef * (Bv[i] * xv[k]));
                acc = fmaf(Cv[i], hs[k][i], acc);
            }
            acc = quad_sum(acc);
            // every lane forms the gated output (so no load sinks into the
            // store's branch); lane q = 0 of the quad stores it
            float yv = acc + skip_on * dsk[k] * xv[k];
            if (z_)
                yv *= silu_hw(zv[k]);
            if (!live[k])
                continue;
            if (q == 0)
                E::store(reinterpret_cast<T *>(y_) + cq[k], yv);
            if constexpr (KC > 1) {
                if (q >= 1 && q < KC)
                    E::store(reinterpret_cast<T *>(conv_state) + cq[k] * (KC - 1) + (q - 1), tu[k]);
            }
            store_state4<NT>(h, gq[k], hs[k]);
        }
    }
}

// Any N <= 16: one lane per channel.
template <bool BF16, int KC, bool NT>
__global__ void __launch_bounds__(kThreads) state_update_kernel(
    float *__restrict__ h, const void *__restrict__ x_, const void *__restrict__ dt_,
    const float *__restrict__ dt_bias, const float *__restrict__ A, const void *__restrict__ Bm_,
    const void *__restrict__ Cm_, const float *__restrict__ Dskip, const void *__restrict__ z_,
    void *__restrict__ y_, int64_t D, int N, int64_t n_ch, void *__restrict__ conv_state,
    const float *__restrict__ conv_w, const float *__restrict__ conv_b)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= n_ch)
        return;
    const int64_t b = c / D, d = c - b * D;
    const T *Bm = reinterpret_cast<const T *>(Bm_) + b * N;
    const T *Cm = reinterpret_cast<const T *>(Cm_) + b * N;
    float xv = E::load(reinterpret_cast<const T *>(x_) + c);
    if constexpr (KC > 0) {
        ConvStep<BF16, KC> cv;
        cv.load(conv_state, xv, conv_w, conv_b ? conv_b : conv_w, c, d);
        xv = cv.out(conv_b ? 1.f : 0.f);
#pragma unroll
        for (int j = 0; j < KC - 1; ++j)
            cv.store_slot(conv_state, c, j);
    }
    const float dtv = E::load(reinterpret_cast<const T *>(dt_) + c);
    const float bias = dt_bias ? dt_bias[d] : 0.f;
    const float l = softplus_log2(fmaf(dtv, kLog2e, bias * kLog2e));  // Δ / ln 2
    const float delta = l * kLn2;
    float acc = 0.f;
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        const float en = hw_exp2(an * l);
        const float coef = zoh_input_coef(an, delta, en);
        const float hn = fmaf(en, load_state<NT>(h + c * N + n), coef * (E::load(Bm + n) * xv));
        store_state<NT>(h + c * N + n, hn);
        acc = fmaf(E::load(Cm + n), hn, acc);
    }
    float yv = acc + (Dskip ? Dskip[d] : 0.f) * xv;
    if (z_)
        yv *= silu_hw(E::load(reinterpret_cast<const T *>(z_) + c));
    E::store(reinterpret_cast<T *>(y_) + c, yv);
}

template <int KC, bool NT>
hipError_t launch_state_update_k(const StepArgs &a, hipStream_t s)
{
    const int64_t n_ch = a.B * a.D;
    const size_t bc_align = a.bf16 ? 8 : 16;
    const bool quad = a.N == kMaxN && ((uintptr_t)a.h % 16) == 0 && ((uintptr_t)a.A % 16) == 0 &&
                      ((uintptr_t)a.Bm % bc_align) == 0 && ((uintptr_t)a.Cm % bc_align) == 0;
    if (quad) {
        constexpr int kQPT = kQuadsPerLane;
        const int64_t per_block = (int64_t)kThreads * kQPT;
        for (int64_t b0 = 0; b0 < a.B; b0 += 65535) {
            const dim3 grid((unsigned)((4 * a.D + per_block - 1) / per_block),
                            (unsigned)min(a.B - b0, (int64_t)65535));
            if (a.bf16)
                hipLaunchKernelGGL((state_update_quad_kernel<true, kQPT, KC, NT>), grid, dim3(kThreads),
                                   0, s, a.h, a.x, a.dt, a.dt_bias, a.A, a.Bm, a.Cm, a.Dskip, a.z,
                                   a.y, b0, a.D, a.conv_state, a.conv_w, a.conv_b);
            else
                hipLaunchKernelGGL((state_update_quad_kernel<false, kQPT, KC, NT>), grid,
                                   dim3(kThreads), 0, s, a.h, a.x, a.dt, a.dt_bias, a.A, a.Bm,
                                   a.Cm, a.Dskip, a.z, a.y, b0, a.D, a.conv_state, a.conv_w,
                                   a.conv_b);
        }
    } else {
        const dim3 grid((unsigned)((n_ch + kThreads - 1) / kThreads));
        if (a.bf16)
            hipLaunchKernelGGL((state_update_kernel<true, KC, NT>), grid, dim3(kThreads), 0, s, a.h,
                               a.x, a.dt, a.dt_bias, a.A, a.Bm, a.Cm, a.Dskip, a.z, a.y, a.D, a.N,
                               n_ch, a.conv_state, a.conv_w, a.conv_b);
        else
            hipLaunchKernelGGL((state_update_kernel<false, KC, NT>), grid, dim3(kThreads), 0, s, a.h,
                               a.x, a.dt, a.dt_bias, a.A, a.Bm, a.Cm, a.Dskip, a.z, a.y, a.D, a.N,
                               n_ch, a.conv_state, a.conv_w, a.conv_b);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const StepArgs &a, hipStream_t s)
{
    if (a.B * a.D == 0)
        return hipSuccess;
    if (a.stream_state) {
        switch (a.conv_K) {
        case 0: return launch_state_update_k<0, true>(a, s);
        case 1: return launch_state_update_k<1, true>(a, s);
        case 2: return launch_state_update_k<2, true>(a, s);
        case 3: return launch_state_update_k<3, true>(a, s);
        case 4: return launch_state_update_k<4, true>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.conv_K) {
    case 0: return launch_state_update_k<0, false>(a, s);
    case 1: return launch_state_update_k<1, false>(a, s);
    case 2: return launch_state_update_k<2, false>(a, s);
    case 3: return launch_state_update_k<3, false>(a, s);
    case 4: return launch_state_update_k<4, false>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mamba
