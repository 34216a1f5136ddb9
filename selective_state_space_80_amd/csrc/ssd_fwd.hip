// Mamba-2 form of the selective scan ("SSD") for gfx950, on the matrix cores.
//
// With one decay value per head (A = a_h times the identity, shared by the
// head's P channels and N states) and B, C shared by a group of heads, the
// map from a head's inputs to its outputs is a structured lower-triangular
// matrix, so the scan can be done with matrix multiplications
// ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式" §4.2).
// Per head and chunk of kQ = 64 steps, with Δ_t = softplus(dt_t + bias),
// ℓ_t = Δ_t a, exact ZOH coefficient β_t = (e^ℓ_t - 1)/a (Δ_t at a = 0), and
// the chunk-local cumulative log decay Λ_t = Σ_{k<=t} ℓ_k:
//   Y_diag[t][p] = Σ_{s<=t} (C_t . B_s) e^(Λ_t - Λ_s) β_s x_s[p]   (within the chunk)
//   Y_off[t][p]  = e^Λ_t Σ_n C_t[n] H[n][p]                        (state entering the chunk)
//   S[n][p]      = Σ_s e^(Λ_end - Λ_s) β_s B_s[n] x_s[p]           (chunk's own contribution)
//   H           <- e^Λ_end H + S
//   out = (Y_diag + Y_off + D x) SiLU(z)
// C.B^T, M.X, C.H and B^T.(w x) run as bf16 MFMAs with fp32 accumulation. The
// operands that are not input values (the scaled chunk matrix M, the state H
// and the scaled x) are split into bf16 hi + lo parts, so they carry about 16
// significant bits; B, C and x are bf16 inputs and exact.
//
// One workgroup (4 waves) per (batch row, head) walks the head's chunks in
// order; wave w owns channels [16w, 16w+16) of the head: their 16 x N slice of
// H lives in its registers in the MFMA accumulator layout, which is also the
// B-operand layout the C.H product needs.
#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kQ = 64;        // chunk length
constexpr int kP = kSsdHeadDim;  // channels per head
constexpr int kT = 256;       // threads per workgroup
constexpr int kQP = kQ + 8;   // row of an s-contiguous bf16 array (16-byte aligned rows)
constexpr int kYP = kP + 1;   // row of the fp32 output tile

// MFMA lane layouts (64 lanes, l16 = lane % 16, g4 = lane / 16), D = A B:
//   16x16x16 bf16: A[l16][4 g4 + j], B[4 g4 + j][l16], j < 4
//   16x16x32 bf16: A[l16][8 g4 + j], B[8 g4 + j][l16], j < 8
//   D (both): lane holds D[4 g4 + i][l16], i < 4
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

// v ≈ hi + lo, both bf16 (round to nearest even)
__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo)
{
    hi = f32_to_bf16_bits(v);
    lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ float bf16_at(const uint4 &v, int j)
{
    const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return bf16_bits_to_f32((j & 1) ? (w >> 16) : (w & 0xffffu));
}

struct SsdKArgs {
    const uint16_t *x, *dt, *Bm, *Cm, *z;
    const float *dt_bias, *A, *Dskip, *h0;
    uint16_t *y;
    float *h_last;
    int64_t B, L, H, G;
};

// causal 16 x 16 tiles (t-block, s-block) of a chunk's 64 x 64 matrix
constexpr int kTiles = 10;
__device__ constexpr int kTB[kTiles] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ constexpr int kSB[kTiles] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int N>
__global__ void __launch_bounds__(kT) ssd_fwd_kernel(SsdKArgs p)
{
    constexpr int NP = N + 8;  // row of an n-contiguous bf16 array
    constexpr int NB = N / 16;
    constexpr size_t kBRegion = (size_t)kQ * NP * 2 + (size_t)N * kQP * 2;
    constexpr size_t kYRegion = (size_t)kQ * kYP * 4;
    constexpr size_t kRegion = kBRegion > kYRegion ? kBRegion : kYRegion;
    __shared__ __align__(16) uint16_t sC[kQ * NP];          // C[t][n]
    __shared__ __align__(16) unsigned char sR[kRegion];     // B[s][n], B^T[n][s]; later Y
    __shared__ __align__(16) uint16_t sXt[kP * kQP];        // x^T[p][s]
    __shared__ __align__(16) uint16_t sXw[2][kP * kQP];     // (w x)^T[p][s], hi and lo
    __shared__ __align__(16) uint16_t sM[kTiles][2][64 * 4];  // M tiles, hi and lo, A layout
    __shared__ float sLam[kQ], sBeta[kQ], sW[kQ], sEL[kQ];
    __shared__ float sDecay;
    uint16_t *sB = reinterpret_cast<uint16_t *>(sR);
    uint16_t *sBt = sB + kQ * NP;
    float *sY = reinterpret_cast<float *>(sR);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh - b * p.H;
    const int64_t grp = h / (p.H / p.G);
    const float a = p.A[h];
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
    const float Dv = p.Dskip ? p.Dskip[h] : 0.f;
    const int pcol = 16 * w + l16;  // this lane's channel in the S, H and Y tiles

    // Hs[nb][i] = H[n = 16 nb + 4 g4 + i][p = pcol]
    float Hs[NB][4];
    {
        const float *h0 = p.h0 ? p.h0 + ((b * p.H + h) * kP + pcol) * N : nullptr;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float4 v = h0 ? *reinterpret_cast<const float4 *>(h0 + 16 * nb + 4 * g4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            Hs[nb][0] = v.x;
            Hs[nb][1] = v.y;
            Hs[nb][2] = v.z;
            Hs[nb][3] = v.w;
        }
    }

    const int64_t n_chunks = (p.L + kQ - 1) / kQ;
    for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t t0 = c * kQ;
        const int nt = (int)min((int64_t)kQ, p.L - t0);

        // ---- 1. stage B (both layouts), C and x^T; steps past L are zero ---
        for (int e = tid; e < kQ * (N / 8); e += kT) {
            const int r = e / (N / 8), c8 = (e % (N / 8)) * 8;
            uint4 vb = make_uint4(0u, 0u, 0u, 0u), vc = vb;
            if (r < nt) {
                const int64_t o = ((b * p.L + t0 + r) * p.G + grp) * N + c8;
                vb = *reinterpret_cast<const uint4 *>(p.Bm + o);
                vc = *reinterpret_cast<const uint4 *>(p.Cm + o);
            }
            *reinterpret_cast<uint4 *>(sB + r * NP + c8) = vb;
            *reinterpret_cast<uint4 *>(sC + r * NP + c8) = vc;
            const uint32_t wv[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sBt[(c8 + 2 * k) * kQP + r] = (uint16_t)(wv[k] & 0xffffu);
                sBt[(c8 + 2 * k + 1) * kQP + r] = (uint16_t)(wv[k] >> 16);
            }
        }
        for (int e = tid; e < kQ * (kP / 8); e += kT) {
            const int r = e / (kP / 8), c8 = (e % (kP / 8)) * 8;
            uint4 vx = make_uint4(0u, 0u, 0u, 0u);
            if (r < nt)
                vx = *reinterpret_cast<const uint4 *>(p.x + ((b * p.L + t0 + r) * p.H + h) * kP + c8);
            const uint32_t wv[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sXt[(c8 + 2 * k) * kQP + r] = (uint16_t)(wv[k] & 0xffffu);
                sXt[(c8 + 2 * k + 1) * kQP + r] = (uint16_t)(wv[k] >> 16);
            }
        }
        // ---- 2. per step (wave 0, lane = step): Δ, ℓ = Δ a, β, Λ ------------
        if (w == 0) {
            float ell = 0.f, beta = 0.f;  // steps past L: no decay, no input
            if (lane < nt) {
                const float v = bf16_bits_to_f32(p.dt[(b * p.L + t0 + lane) * p.H + h]) + bias;
                const float delta = softplus_log2(v * kLog2e) * kLn2;
                ell = delta * a;
                beta = zoh_input_coef(a, delta, hw_exp2(ell * kLog2e));
            }
            float cum = ell;  // inclusive prefix sum over the chunk
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(cum, off);
                if (lane >= off)
                    cum += o;
            }
            const float lend = __shfl(cum, 63);
            sLam[lane] = cum;
            sBeta[lane] = beta;
            sW[lane] = hw_exp2((lend - cum) * kLog2e) * beta;
            sEL[lane] = hw_exp2(cum * kLog2e);
            if (lane == 0)
                sDecay = hw_exp2(lend * kLog2e);
        }
        __syncthreads();

        // ---- 3. w_s x_s[p] split into bf16 hi + lo, s-contiguous ------------
        for (int e = tid; e < kP * (kQ / 2); e += kT) {
            const int pp = e / (kQ / 2), s2 = (e % (kQ / 2)) * 2;
            const uint32_t xv = *reinterpret_cast<const uint32_t *>(sXt + pp * kQP + s2);
            uint32_t h0b, l0b, h1b, l1b;
            split_bf16(bf16_bits_to_f32(xv & 0xffffu) * sW[s2], h0b, l0b);
            split_bf16(bf16_bits_to_f32(xv >> 16) * sW[s2 + 1], h1b, l1b);
            *reinterpret_cast<uint32_t *>(sXw[0] + pp * kQP + s2) = pack2(h0b, h1b);
            *reinterpret_cast<uint32_t *>(sXw[1] + pp * kQP + s2) = pack2(l0b, l1b);
        }
        // ---- 4. causal tiles M^T[s][t] = (B_s . C_t) e^(Λ_t - Λ_s) β_s, s <= t
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            if (k % 4 != w)
                continue;
            const int tb = kTB[k], sb = kSB[k];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (N % 32 == 0) {
#pragma unroll
                for (int n0 = 0; n0 < N; n0 += 32) {
                    const bf16x8 av =
                        *reinterpret_cast<const bf16x8 *>(sB + (16 * sb + l16) * NP + n0 + 8 * g4);
                    const bf16x8 bv =
                        *reinterpret_cast<const bf16x8 *>(sC + (16 * tb + l16) * NP + n0 + 8 * g4);
                    acc = mma32(av, bv, acc);
                }
            } else {
#pragma unroll
                for (int n0 = 0; n0 < N; n0 += 16) {
                    const s16x4 av =
                        *reinterpret_cast<const s16x4 *>(sB + (16 * sb + l16) * NP + n0 + 4 * g4);
                    const s16x4 bv =
                        *reinterpret_cast<const s16x4 *>(sC + (16 * tb + l16) * NP + n0 + 4 * g4);
                    acc = mma16(av, bv, acc);
                }
            }
            // lane: G^T[s = 16 sb + 4 g4 + i][t = 16 tb + l16]
            const int t = 16 * tb + l16;
            const float lt = sLam[t];
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * sb + 4 * g4 + i;
                const float m =
                    s <= t ? acc[i] * hw_exp2((lt - sLam[s]) * kLog2e) * sBeta[s] : 0.f;
                split_bf16(m, hi[i], lo[i]);
            }
            *reinterpret_cast<uint2 *>(&sM[k][0][lane * 4]) =
                make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
            *reinterpret_cast<uint2 *>(&sM[k][1][lane * 4]) =
                make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
        }
        __syncthreads();

        // ---- 5. this wave's channels: Y = M x + e^Λ C H, S = B^T (w x) -----
        f32x4 yd[4], yo[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            yd[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            yo[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            const int tb = kTB[k], sb = kSB[k];
            const s16x4 mh = *reinterpret_cast<const s16x4 *>(&sM[k][0][lane * 4]);
            const s16x4 ml = *reinterpret_cast<const s16x4 *>(&sM[k][1][lane * 4]);
            const s16x4 xv = *reinterpret_cast<const s16x4 *>(sXt + pcol * kQP + 16 * sb + 4 * g4);
            yd[tb] = mma16(mh, xv, yd[tb]);
            yd[tb] = mma16(ml, xv, yd[tb]);
        }
        // H as bf16 hi / lo pairs: Hh[nb][0] = (n, n+1), Hh[nb][1] = (n+2, n+3), n = 16 nb + 4 g4
        uint32_t Hh[NB][2], Hl[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                split_bf16(Hs[nb][i], hi[i], lo[i]);
            Hh[nb][0] = pack2(hi[0], hi[1]);
            Hh[nb][1] = pack2(hi[2], hi[3]);
            Hl[nb][0] = pack2(lo[0], lo[1]);
            Hl[nb][1] = pack2(lo[2], lo[3]);
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const uint16_t *crow = sC + (16 * tb + l16) * NP + 4 * g4;
            if constexpr (NB % 2 == 0) {
                // k slot j of lane group g4: n = 16 nb + 4 g4 + j (j < 4), then
                // 16 (nb+1) + 4 g4 + j - 4: the same relabelling of n on both sides
#pragma unroll
                for (int nb = 0; nb < NB; nb += 2) {
                    const uint2 c0 = *reinterpret_cast<const uint2 *>(crow + 16 * nb);
                    const uint2 c1 = *reinterpret_cast<const uint2 *>(crow + 16 * (nb + 1));
                    const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
                    const bf16x8 bhi = __builtin_bit_cast(
                        bf16x8, make_uint4(Hh[nb][0], Hh[nb][1], Hh[nb + 1][0], Hh[nb + 1][1]));
                    const bf16x8 blo = __builtin_bit_cast(
                        bf16x8, make_uint4(Hl[nb][0], Hl[nb][1], Hl[nb + 1][0], Hl[nb + 1][1]));
                    yo[tb] = mma32(av, bhi, yo[tb]);
                    yo[tb] = mma32(av, blo, yo[tb]);
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const s16x4 av = *reinterpret_cast<const s16x4 *>(crow + 16 * nb);
                    const s16x4 bhi = __builtin_bit_cast(s16x4, make_uint2(Hh[nb][0], Hh[nb][1]));
                    const s16x4 blo = __builtin_bit_cast(s16x4, make_uint2(Hl[nb][0], Hl[nb][1]));
                    yo[tb] = mma16(av, bhi, yo[tb]);
                    yo[tb] = mma16(av, blo, yo[tb]);
                }
            }
        }
        f32x4 sa[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            sa[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < kQ; s0 += 32) {
                const bf16x8 av =
                    *reinterpret_cast<const bf16x8 *>(sBt + (16 * nb + l16) * kQP + s0 + 8 * g4);
                const bf16x8 xh =
                    *reinterpret_cast<const bf16x8 *>(sXw[0] + pcol * kQP + s0 + 8 * g4);
                const bf16x8 xl =
                    *reinterpret_cast<const bf16x8 *>(sXw[1] + pcol * kQP + s0 + 8 * g4);
                sa[nb] = mma32(av, xh, sa[nb]);
                sa[nb] = mma32(av, xl, sa[nb]);
            }
        }
        __syncthreads();  // every wave is done with B before Y takes its place

        // ---- 6. Y to LDS, state update, then gate and store -----------------
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * g4 + i;
                sY[t * kYP + pcol] = fmaf(sEL[t], yo[tb][i], yd[tb][i]);
            }
        }
        const float decay = sDecay;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Hs[nb][i] = fmaf(decay, Hs[nb][i], sa[nb][i]);
        }
        __syncthreads();
        {
            const int t = tid >> 2, pp = (tid & 3) * 16;  // 16 channels of one step
            if (t < nt) {
                const int64_t o = ((b * p.L + t0 + t) * p.H + h) * kP + pp;
                const uint4 x0 = *reinterpret_cast<const uint4 *>(p.x + o);
                const uint4 x1 = *reinterpret_cast<const uint4 *>(p.x + o + 8);
                uint4 z0 = make_uint4(0u, 0u, 0u, 0u), z1 = z0;
                if (p.z) {
                    z0 = *reinterpret_cast<const uint4 *>(p.z + o);
                    z1 = *reinterpret_cast<const uint4 *>(p.z + o + 8);
                }
                uint32_t out[8];
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const uint4 &xs = j < 8 ? x0 : x1;
                    const uint4 &zs = j < 8 ? z0 : z1;
                    float v0 = fmaf(Dv, bf16_at(xs, j & 7), sY[t * kYP + pp + j]);
                    float v1 = fmaf(Dv, bf16_at(xs, (j & 7) + 1), sY[t * kYP + pp + j + 1]);
                    if (p.z) {
                        v0 *= silu_hw(bf16_at(zs, j & 7));
                        v1 *= silu_hw(bf16_at(zs, (j & 7) + 1));
                    }
                    out[j / 2] = pack2(f32_to_bf16_bits(v0), f32_to_bf16_bits(v1));
                }
                *reinterpret_cast<uint4 *>(p.y + o) = make_uint4(out[0], out[1], out[2], out[3]);
                *reinterpret_cast<uint4 *>(p.y + o + 8) = make_uint4(out[4], out[5], out[6], out[7]);
            }
        }
        __syncthreads();  // Y's LDS is B's again for the next chunk
    }
    if (p.h_last) {
        float *hl = p.h_last + ((b * p.H + h) * kP + pcol) * N;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<float4 *>(hl + 16 * nb + 4 * g4) =
                make_float4(Hs[nb][0], Hs[nb][1], Hs[nb][2], Hs[nb][3]);
    }
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdArgs &a, hipStream_t s)
{
    SsdKArgs k;
    k.x = static_cast<const uint16_t *>(a.x);
    k.dt = static_cast<const uint16_t *>(a.dt);
    k.Bm = static_cast<const uint16_t *>(a.Bm);
    k.Cm = static_cast<const uint16_t *>(a.Cm);
    k.z = static_cast<const uint16_t *>(a.z);
    k.dt_bias = a.dt_bias;
    k.A = a.A;
    k.Dskip = a.Dskip;
    k.h0 = a.h0;
    k.y = static_cast<uint16_t *>(a.y);
    k.h_last = a.h_last;
    k.B = a.B;
    k.L = a.L;
    k.H = a.H;
    k.G = a.G;
    const dim3 grid((unsigned)(a.B * a.H)), block(kT);
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, s);
    switch (a.N) {
    case 16: hipLaunchKernelGGL(ssd_fwd_kernel<16>, grid, block, 0, s, k); break;
    case 32: hipLaunchKernelGGL(ssd_fwd_kernel<32>, grid, block, 0, s, k); break;
    case 64: hipLaunchKernelGGL(ssd_fwd_kernel<64>, grid, block, 0, s, k); break;
    case 128: hipLaunchKernelGGL(ssd_fwd_kernel<128>, grid, block, 0, s, k); break;
    default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (a.ev_stop)
        (void)hipEventRecord(a.ev_stop, s);
    return e;
}

}  // namespace mamba
