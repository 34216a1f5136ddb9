// Causal depthwise conv1d + SiLU for gfx950: the front end of the Mamba block
// ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式" §3.1: a causal
// Conv1D supplies local context before the selective SSM; kernel size 4 per
// "Mamba架构与SSM模型：高效序列建模技术解析" §3.2).
//   out[b,d,t] = SiLU(bias_d + sum_{k<K} w[d,k] x[b,d,t-(K-1)+k]),  x[t<0] = 0
// Streaming and HBM-bound (one read, one write per element): each thread makes
// the outputs of one 16-byte piece of a row (8 bf16 or 4 fp32 values), so
// consecutive lanes read and write consecutive pieces and every load or store
// instruction of a wave covers one contiguous kilobyte.  The left halo (K - 1
// inputs) is the previous one or two pieces, which the neighbouring threads
// load too, so it comes from cache, not HBM.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

// One 16-byte piece of a row: 8 bf16 or 4 fp32 values.
template <bool BF16> constexpr int kPiece = BF16 ? 8 : 4;

template <bool BF16>
__device__ __forceinline__ void load_piece(const void *base, int64_t off, float (&v)[kPiece<BF16>])
{
    if constexpr (!BF16) {
        const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
        const uint4 a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + off);
        const uint32_t w4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w4[k] << 16);
            v[2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void store_piece(void *base, int64_t off, const float (&v)[kPiece<BF16>])
{
    if constexpr (!BF16) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(base) + off) =
            make_float4(v[0], v[1], v[2], v[3]);
    } else {
        uint32_t w4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w4[k] = cvt2(v[2 * k], v[2 * k + 1]);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(base) + off) =
            make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
}

// Rows of whole 16-byte pieces (L a multiple of the piece, 16-byte aligned).
// Grid (D, pieces / 256, B): the workgroup's channel and batch row come from
// its indices (no division; the weights are the same for the whole
// workgroup), thread t makes the outputs of piece 256 blockIdx.y + t.  Its
// halo pieces are loaded unconditionally (a piece at the start of a row reads
// itself) and zeroed where they would lie before the row.
template <bool BF16, int K>
__global__ void __launch_bounds__(256) conv1d_silu_piece_kernel(
    const void *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    void *__restrict__ out, int64_t D, int64_t L)
{
    constexpr int V = kPiece<BF16>;
    constexpr int HP = (K - 1 + V - 1) / V;  // halo pieces
    const int64_t t0 = ((int64_t)blockIdx.y * 256 + threadIdx.x) * V;
    if (t0 >= L)
        return;
    const int64_t d = blockIdx.x;
    const int64_t base = ((int64_t)blockIdx.z * D + d) * L;
    const float bias_raw = (bias ? bias : w)[d];
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        wk[k] = w[d * K + k];
    float win[(HP + 1) * V];  // x[t0 - HP V .. t0 + V - 1]
    {
        float v[V];
        load_piece<BF16>(x, base + t0, v);
#pragma unroll
        for (int k = 0; k < V; ++k)
            win[HP * V + k] = v[k];
    }
#pragma unroll
    for (int h = 1; h <= HP; ++h) {
        float v[V];
        const bool in_row = t0 >= h * V;
        load_piece<BF16>(x, base + (in_row ? t0 - h * V : t0), v);
#pragma unroll
        for (int k = 0; k < V; ++k)
            win[(HP - h) * V + k] = in_row ? v[k] : 0.f;
    }
    const float bv = bias ? bias_raw : 0.f;
    float res[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        // tap k multiplies x[t0 + j - (K-1) + k]
        float acc = bv;
#pragma unroll
        for (int k = 0; k < K; ++k)
            acc = fmaf(wk[k], win[HP * V + j - (K - 1) + k], acc);
        res[j] = silu_hw(acc);
    }
    store_piece<BF16>(out, base + t0, res);
}

// Other rows (L not a multiple of the piece, or unaligned): kVT outputs per
// thread, element loads with bounds checks.
constexpr int kVT = 8;

template <bool BF16, int K>
__global__ void __launch_bounds__(256) conv1d_silu_kernel(
    const void *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    void *__restrict__ out, int64_t D, int64_t L, int64_t vec_per_row, int64_t n_threads)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_threads)
        return;
    const int64_t row = i / vec_per_row;  // b * D + d
    const int64_t t0 = (i - row * vec_per_row) * kVT;
    const int64_t d = row % D;
    const int64_t base = row * L;

    float win[2 * kVT];  // x[t0-8 .. t0+7]
    const T *xr = reinterpret_cast<const T *>(x) + base;
#pragma unroll
    for (int k = 0; k < 2 * kVT; ++k) {
        const int64_t t = t0 - kVT + k;
        win[k] = (t >= 0 && t < L) ? E::load(xr + t) : 0.f;
    }

    const float bv = bias ? bias[d] : 0.f;
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        wk[k] = w[d * K + k];
    T *orow = reinterpret_cast<T *>(out) + base;
#pragma unroll
    for (int j = 0; j < kVT; ++j) {
        // tap k multiplies x[t - (K-1) + k], i.e. window index kVT + j - (K-1) + k
        float acc = bv;
#pragma unroll
        for (int k = 0; k < K; ++k)
            acc = fmaf(wk[k], win[kVT + j - (K - 1) + k], acc);
        if (t0 + j < L)
            E::store(orow + t0 + j, silu_hw(acc));
    }
}

template <bool BF16, int K>
hipError_t launch_typed(const ConvArgs &a, hipStream_t s)
{
    constexpr int V = kPiece<BF16>;
    const int64_t piece_blocks = (a.L / V + 255) / 256;
    if (a.L % V == 0 && (((uintptr_t)a.x | (uintptr_t)a.out) % 16 == 0) && a.B <= 65535 &&
        piece_blocks <= 65535 && a.D < (int64_t(1) << 24)) {  // D x 256 work-items < 2^32
        hipLaunchKernelGGL((conv1d_silu_piece_kernel<BF16, K>),
                           dim3((unsigned)a.D, (unsigned)piece_blocks, (unsigned)a.B), dim3(256), 0,
                           s, a.x, a.w, a.bias, a.out, a.D, a.L);
        return hipGetLastError();
    }
    const int64_t vpr = (a.L + kVT - 1) / kVT;
    const int64_t n = a.B * a.D * vpr;
    hipLaunchKernelGGL((conv1d_silu_kernel<BF16, K>), dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, a.x, a.w, a.bias, a.out, a.D, a.L, vpr, n);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_k(const ConvArgs &a, hipStream_t s)
{
    switch (a.K) {
    case 1: return launch_typed<BF16, 1>(a, s);
    case 2: return launch_typed<BF16, 2>(a, s);
    case 3: return launch_typed<BF16, 3>(a, s);
    case 4: return launch_typed<BF16, 4>(a, s);
    case 5: return launch_typed<BF16, 5>(a, s);
    case 6: return launch_typed<BF16, 6>(a, s);
    case 7: return launch_typed<BF16, 7>(a, s);
    case 8: return launch_typed<BF16, 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// Decode step of the front end: one new input per channel, the K-1 previous
// raw inputs carried in `state` ([B, D, K-1], oldest first).
//   out[b,d] = SiLU(bias_d + sum_{k<K-1} w[d,k] state[b,d,k] + w[d,K-1] x[b,d])
//   state[b,d,:] <- (state[b,d,1:], x[b,d])
// One thread per channel on a (channel block, batch row) grid, so no thread
// divides; the window is read whole before the state moves by one slot in
// place.
template <bool BF16, int K>
__global__ void __launch_bounds__(256) conv1d_update_kernel(void *__restrict__ state_,
                                                            const void *__restrict__ x_,
                                                            const float *__restrict__ w,
                                                            const float *__restrict__ bias,
                                                            void *__restrict__ out_, int64_t D,
                                                            int64_t b0)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (d >= D)
        return;
    const int64_t i = (b0 + blockIdx.y) * D + d;
    T *state = reinterpret_cast<T *>(state_) + i * (K - 1);
    T win[K];  // the K inputs of this step, oldest first
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
        win[k] = state[k];
    win[K - 1] = reinterpret_cast<const T *>(x_)[i];
    const float bias_raw = (bias ? bias : w)[d];
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        wk[k] = w[d * K + k];
    float acc = bias ? bias_raw : 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k)
        acc = fmaf(wk[k], E::load(&win[k]), acc);
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
        state[k] = win[k + 1];
    E::store(reinterpret_cast<T *>(out_) + i, silu_hw(acc));
}

// The same step for rows of whole pieces: thread t owns the C channels of one
// 16-byte piece of x (C = 8 bf16 or 4 fp32).  Their windows are C (K-1)
// consecutive state values, i.e. K-1 whole pieces, and their weights C K
// consecutive floats, so every access is a 16-byte one and each wave's loads
// and stores cover contiguous runs.  Needs D a multiple of C and 16-byte
// aligned state, x, out, w (and bias).
template <bool BF16, int K>
__global__ void __launch_bounds__(256) conv1d_update_piece_kernel(void *__restrict__ state_,
                                                                  const void *__restrict__ x_,
                                                                  const float *__restrict__ w,
                                                                  const float *__restrict__ bias,
                                                                  void *__restrict__ out_,
                                                                  int64_t D, int64_t b0)
{
    constexpr int C = kPiece<BF16>;
    const int64_t d0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * C;
    if (d0 >= D)
        return;
    const int64_t i0 = (b0 + blockIdx.y) * D + d0;  // flat index of the first channel
    float st[(K - 1) * C + 1];  // channel c's window at c (K-1) .. c (K-1) + K-2
#pragma unroll
    for (int q = 0; q < K - 1; ++q) {
        float v[C];
        load_piece<BF16>(state_, i0 * (K - 1) + q * C, v);
#pragma unroll
        for (int k = 0; k < C; ++k)
            st[q * C + k] = v[k];
    }
    float xv[C];
    load_piece<BF16>(x_, i0, xv);
    float wv[C * K];
#pragma unroll
    for (int q = 0; q < C * K / 4; ++q) {
        const float4 a = reinterpret_cast<const float4 *>(w + d0 * K)[q];
        wv[4 * q] = a.x; wv[4 * q + 1] = a.y; wv[4 * q + 2] = a.z; wv[4 * q + 3] = a.w;
    }
    float bv[C];
#pragma unroll
    for (int q = 0; q < C / 4; ++q) {
        const float4 a = reinterpret_cast<const float4 *>((bias ? bias : w) + d0)[q];
        bv[4 * q] = a.x; bv[4 * q + 1] = a.y; bv[4 * q + 2] = a.z; bv[4 * q + 3] = a.w;
    }
    float res[C], ns[(K - 1) * C + 1];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        float acc = bias ? bv[c] : 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k)
            acc = fmaf(wv[c * K + k], k < K - 1 ? st[c * (K - 1) + k] : xv[c], acc);
        res[c] = silu_hw(acc);
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
            ns[c * (K - 1) + j] = j < K - 2 ? st[c * (K - 1) + j + 1] : xv[c];
    }
#pragma unroll
    for (int q = 0; q < K - 1; ++q) {
        float v[C];
#pragma unroll
        for (int k = 0; k < C; ++k)
            v[k] = ns[q * C + k];
        store_piece<BF16>(state_, i0 * (K - 1) + q * C, v);
    }
    store_piece<BF16>(out_, i0, res);
}

template <bool BF16, int K>
hipError_t launch_update_typed(const ConvUpdateArgs &a, hipStream_t s)
{
    constexpr int C = kPiece<BF16>;
    const bool pieces = a.D % C == 0 &&
                        (((uintptr_t)a.state | (uintptr_t)a.x | (uintptr_t)a.out |
                          (uintptr_t)a.w | (uintptr_t)a.bias) % 16) == 0;
    const unsigned gx = (unsigned)((pieces ? a.D / C + 255 : a.D + 255) / 256);
    for (int64_t b0 = 0; b0 < a.B; b0 += 65535) {
        const unsigned gy = (unsigned)std::min<int64_t>(a.B - b0, 65535);
        if (pieces)
            hipLaunchKernelGGL((conv1d_update_piece_kernel<BF16, K>), dim3(gx, gy), dim3(256), 0,
                               s, a.state, a.x, a.w, a.bias, a.out, a.D, b0);
        else
            hipLaunchKernelGGL((conv1d_update_kernel<BF16, K>), dim3(gx, gy), dim3(256), 0, s,
                               a.state, a.x, a.w, a.bias, a.out, a.D, b0);
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_update_k(const ConvUpdateArgs &a, hipStream_t s)
{
    switch (a.K) {
    case 1: return launch_update_typed<BF16, 1>(a, s);
    case 2: return launch_update_typed<BF16, 2>(a, s);
    case 3: return launch_update_typed<BF16, 3>(a, s);
    case 4: return launch_update_typed<BF16, 4>(a, s);
    case 5: return launch_update_typed<BF16, 5>(a, s);
    case 6: return launch_update_typed<BF16, 6>(a, s);
    case 7: return launch_update_typed<BF16, 7>(a, s);
    case 8: return launch_update_typed<BF16, 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_conv1d_update(const ConvUpdateArgs &a, hipStream_t s)
{
    if (a.B * a.D == 0)
        return hipSuccess;
    return a.bf16 ? launch_update_k<true>(a, s) : launch_update_k<false>(a, s);
}

hipError_t launch_conv1d_silu(const ConvArgs &a, hipStream_t s)
{
    if (a.B * a.D * a.L == 0)
        return hipSuccess;
    return a.bf16 ? launch_k<true>(a, s) : launch_k<false>(a, s);
}

}  // namespace mamba
