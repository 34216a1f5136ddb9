// Mamba-2 form of the selective scan ("SSD") for gfx950, on the matrix cores.
//
// With one decay value per head (A = a_h times the identity, shared by the
// head's P channels and N states) and B, C shared by a group of heads, the
// map from a head's inputs to its outputs is a structured lower-triangular
// matrix, so the scan can be done with matrix multiplications
// ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式" §4.2).
// Per head and chunk of Q steps (32 or 64), with Δ_t = softplus(dt_t + bias),
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

constexpr int kP = kSsdHeadDim;  // channels per head
constexpr int kT = 256;       // threads per workgroup
// row of the fp32 output tile: 16-byte rows whose stride (68 words) puts the
// two 16-lane halves of a store of step 6 on different banks
constexpr int kYP = kP + 4;

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

// (a, b) ≈ hi + lo, each a packed bf16 pair: hi the rounded values, lo the
// rounded remainders
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = cvt2(a, b);
    lo = cvt2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// v + (v of the lane that DPP control CTRL selects, in the rows of ROW_MASK;
// 0 where there is none)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + __int_as_float(
                   __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

struct SsdKArgs {
    const uint16_t *x, *dt, *Bm, *Cm, *z;
    const float *dt_bias, *A, *Dskip, *h0;
    uint16_t *y;
    float *h_last;
    int64_t B, L, H, G;
};

// The causal 16 x 16 tiles (t-block, s-block), s-block <= t-block, of a
// chunk's Q x Q matrix, numbered row by row: k -> (tile_tb(k), tile_sb(k)).
__host__ __device__ constexpr int tile_tb(int k)
{
    int tb = 0;
    while ((tb + 1) * (tb + 2) / 2 <= k)
        ++tb;
    return tb;
}
__host__ __device__ constexpr int tile_sb(int k) { return k - tile_tb(k) * (tile_tb(k) + 1) / 2; }

// chunk length per state size: 32-step chunks keep the workgroup's LDS and
// registers small enough for three workgroups per CU where N allows
template <int N> constexpr int ssd_chunk() { return N == 16 ? 64 : 32; }

template <int N, int Q>
__global__ void __launch_bounds__(kT, (Q == 32 && N <= 64) ? 3 : 2) ssd_fwd_kernel(SsdKArgs p)
{
    constexpr int kQ = Q;               // chunk length
    constexpr int kQP = Q + 8;          // row of an s-contiguous bf16 array (16-byte aligned rows)
    constexpr int TB = Q / 16;          // 16-step blocks per chunk
    constexpr int kTiles = TB * (TB + 1) / 2;
    constexpr int kXPer = Q * kP / kT;  // x, z, y values per thread (one step, kXPer channels)
    constexpr int NP = N + 8;           // row of an n-contiguous bf16 array
    constexpr int NB = N / 16;
    constexpr int kPer = (kQ * N / 8 + kT - 1) / kT;  // 16-byte B, C pieces per thread
    constexpr int kBtPer = kQ * N / kT;               // B^T values per thread
    constexpr int kSW = 3;  // wave with the fewest causal tiles (tile k goes to wave k % 4)
    static_assert(kBtPer % 4 == 0 && kXPer % 8 == 0, "whole 8-byte / 16-byte pieces");
    __shared__ __align__(16) uint16_t sC[kQ * NP];         // C[t][n]
    __shared__ __align__(16) uint16_t sB[kQ * NP];         // B[s][n]
    __shared__ __align__(16) uint16_t sBt[N * kQP];        // B^T[n][s]
    __shared__ __align__(16) uint16_t sX[kQ * (kP + 8)];   // x[s][p]
    __shared__ __align__(16) uint16_t sXt[kP * kQP];       // x^T[p][s]
    __shared__ __align__(16) uint16_t sXw[2][kP * kQP];    // (w x)^T[p][s], hi and lo
    __shared__ __align__(16) float sY[kQ * kYP];           // output tile Y[t][p]
    __shared__ __align__(16) uint16_t sM[kTiles][2][64 * 4];  // M tiles, hi and lo, A layout
    // per step of a chunk: Λ, β, w = e^(Λ_end - Λ) β, e^Λ, and the chunk's
    // e^Λ_end; two buffers, chunks alternate (see step 4)
    __shared__ float sLam[2][kQ], sBeta[2][kQ], sW[2][kQ], sEL[2][kQ];
    __shared__ float sDecay[2];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh - b * p.H;
    const int64_t grp = h / (p.H / p.G);
    const float a = p.A[h];
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
    const float Dv = p.Dskip ? p.Dskip[h] : 0.f;
    const int pcol = 16 * w + l16;  // this lane's channel in the S, H and Y tiles
    const int64_t tstride = p.H * kP;  // x, z, y: elements between consecutive steps

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

    // Global loads of chunk c+1 are issued while chunk c is computed: per
    // thread, B and C rows as 16-byte pieces e = tid + k kT, and x and z as the
    // two 16-byte pieces of step xr, channels xc .. xc+15 (the step and
    // channels this thread gates and stores); wave kSW lane t: dt of step t,
    // first, so that its wait does not include the others.
    // Steps past L load nothing and stage zeros.  Offsets within a chunk are
    // 32-bit (the entry point bounds H P kQ below 2^31).
    constexpr int kXP = kP + 8;  // row of the staged x[s][p]
    uint4 pB[kPer], pC[kPer], pX[kXPer / 8], pZ[kXPer / 8];
    uint32_t pdt = 0;
    const int btn = tid % N, bts = (tid / N) * kBtPer;  // this thread's B^T column and steps
    const int xr = tid / (kP / kXPer), xc = (tid % (kP / kXPer)) * kXPer;
    const int gN = (int)(p.G * N), ts = (int)tstride;
    auto load_chunk = [&](int64_t cc) {
        const int64_t tc = cc * kQ;
        const int ncur = (int)min((int64_t)kQ, p.L - tc);
        const uint16_t *Bb = p.Bm + ((b * p.L + tc) * p.G + grp) * N;
        const uint16_t *Cb = p.Cm + ((b * p.L + tc) * p.G + grp) * N;
        if (w == kSW && lane < ncur)
            pdt = p.dt[(b * p.L + tc + lane) * p.H + h];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int e = tid + k * kT;
            const int r = e / (N / 8), c8 = (e % (N / 8)) * 8;
            pB[k] = pC[k] = make_uint4(0u, 0u, 0u, 0u);
            if (e < kQ * N / 8 && r < ncur) {
                pB[k] = *reinterpret_cast<const uint4 *>(Bb + (r * gN + c8));
                pC[k] = *reinterpret_cast<const uint4 *>(Cb + (r * gN + c8));
            }
        }
        const int64_t xo = ((b * p.L + tc) * p.H + h) * kP;
#pragma unroll
        for (int k = 0; k < kXPer / 8; ++k)
            pX[k] = pZ[k] = make_uint4(0u, 0u, 0u, 0u);
        if (xr < ncur) {
            const int off = xr * ts + xc;
#pragma unroll
            for (int k = 0; k < kXPer / 8; ++k) {
                pX[k] = *reinterpret_cast<const uint4 *>(p.x + xo + off + 8 * k);
                if (p.z)
                    pZ[k] = *reinterpret_cast<const uint4 *>(p.z + xo + off + 8 * k);
            }
        }
    };

    // Step values of a chunk (wave kSW, lane = step): Δ, ℓ = Δ a, β and the
    // chunk-local inclusive prefix Λ of ℓ (DPP within rows of 16, then row
    // broadcasts), into buffer buf.  Steps past L: no decay, no input.
    auto step_values = [&](int buf, uint32_t dtb, int ncur) {
        float ell = 0.f, beta = 0.f;
        if (lane < ncur) {
            const float v = bf16_bits_to_f32(dtb) + bias;
            const float delta = softplus_log2(v * kLog2e) * kLn2;
            ell = delta * a;
            beta = zoh_input_coef(a, delta, hw_exp2(ell * kLog2e));
        }
        float cum = ell;
        cum = dpp_add<0x111, 0xf>(cum);  // row_shr:1
        cum = dpp_add<0x112, 0xf>(cum);  // row_shr:2
        cum = dpp_add<0x114, 0xf>(cum);  // row_shr:4
        cum = dpp_add<0x118, 0xf>(cum);  // row_shr:8
        cum = dpp_add<0x142, 0xa>(cum);  // row_bcast:15 into rows 1 and 3
        if constexpr (kQ > 32)
            cum = dpp_add<0x143, 0xc>(cum);  // row_bcast:31 into rows 2 and 3
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), kQ - 1));
        if (lane < kQ) {
            sLam[buf][lane] = cum;
            sBeta[buf][lane] = beta;
            sW[buf][lane] = hw_exp2((lend - cum) * kLog2e) * beta;
            sEL[buf][lane] = hw_exp2(cum * kLog2e);
        }
        if (lane == 0)
            sDecay[buf] = hw_exp2(lend * kLog2e);
    };

    const int64_t n_chunks = (p.L + kQ - 1) / kQ;
    if (n_chunks > 0) {
        load_chunk(0);
        if (w == kSW)
            step_values(0, pdt, (int)min((int64_t)kQ, p.L));
    }
    for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t t0 = c * kQ;
        const int nt = (int)min((int64_t)kQ, p.L - t0);

        // ---- 1. stage B, C, B^T, x^T from the registers ---------------------
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int e = tid + k * kT;
            if (e < kQ * N / 8) {
                const int r = e / (N / 8), c8 = (e % (N / 8)) * 8;
                *reinterpret_cast<uint4 *>(sB + r * NP + c8) = pB[k];
                *reinterpret_cast<uint4 *>(sC + r * NP + c8) = pC[k];
            }
        }
        uint4 cX[kXPer / 8], cZ[kXPer / 8];  // kept for this thread's skip and gate
#pragma unroll
        for (int k = 0; k < kXPer / 8; ++k) {
            *reinterpret_cast<uint4 *>(sX + xr * kXP + xc + 8 * k) = pX[k];
            cX[k] = pX[k];
            cZ[k] = pZ[k];
        }
        if (c + 1 < n_chunks)
            load_chunk(c + 1);
        const int buf = (int)(c & 1);
        const float *cLam = sLam[buf], *cBeta = sBeta[buf], *cW = sW[buf], *cEL = sEL[buf];
        __syncthreads();

        // ---- 3. transposes: x^T, (w x)^T split into bf16 hi + lo, and B^T ----
        {
            // lane = channel, wave w = steps kQ/4 w .. kQ/4 (w+1) - 1: column
            // reads of x, 16-byte row stores of the transposes
            constexpr int kS = kQ / 4;
            uint32_t xs[kS / 2], hs[kS / 2], ls[kS / 2];
#pragma unroll
            for (int j = 0; j < kS; j += 2) {
                const int s0 = kS * w + j;
                const uint32_t x0 = sX[s0 * kXP + lane], x1 = sX[(s0 + 1) * kXP + lane];
                xs[j / 2] = x0 | (x1 << 16);
                split2(__uint_as_float(x0 << 16) * cW[s0], __uint_as_float(x1 << 16) * cW[s0 + 1],
                       hs[j / 2], ls[j / 2]);
            }
            uint16_t *xt = sXt + lane * kQP + kS * w;
            uint16_t *wh = sXw[0] + lane * kQP + kS * w, *wl = sXw[1] + lane * kQP + kS * w;
#pragma unroll
            for (int c8 = 0; c8 < kS; c8 += 8) {
                const int q = c8 / 2;
                *reinterpret_cast<uint4 *>(xt + c8) = make_uint4(xs[q], xs[q + 1], xs[q + 2], xs[q + 3]);
                *reinterpret_cast<uint4 *>(wh + c8) = make_uint4(hs[q], hs[q + 1], hs[q + 2], hs[q + 3]);
                *reinterpret_cast<uint4 *>(wl + c8) = make_uint4(ls[q], ls[q + 1], ls[q + 2], ls[q + 3]);
            }
            // B^T: column btn, steps bts .. bts + kBtPer - 1 (kBtPer = N/4 >= 4)
#pragma unroll
            for (int j = 0; j < kBtPer; j += 4) {
                const uint32_t b0 = sB[(bts + j) * NP + btn], b1 = sB[(bts + j + 1) * NP + btn];
                const uint32_t b2 = sB[(bts + j + 2) * NP + btn], b3 = sB[(bts + j + 3) * NP + btn];
                *reinterpret_cast<uint2 *>(sBt + btn * kQP + bts + j) =
                    make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            }
        }
        // ---- 4. causal tiles M^T[s][t] = (B_s . C_t) e^(Λ_t - Λ_s) β_s, s <= t
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            if (k % 4 != w)
                continue;
            const int tb = tile_tb(k), sb = tile_sb(k);
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
            const float lt = cLam[t];
            float m[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * sb + 4 * g4 + i;
                m[i] = s <= t ? acc[i] * hw_exp2((lt - cLam[s]) * kLog2e) * cBeta[s] : 0.f;
            }
            uint32_t hi0, lo0, hi1, lo1;
            split2(m[0], m[1], hi0, lo0);
            split2(m[2], m[3], hi1, lo1);
            *reinterpret_cast<uint2 *>(&sM[k][0][lane * 4]) = make_uint2(hi0, hi1);
            *reinterpret_cast<uint2 *>(&sM[k][1][lane * 4]) = make_uint2(lo0, lo1);
        }
        // The step values of the next chunk, by the wave with the fewest tiles
        // (none for 32-step chunks), into the other buffer: its last readers
        // finished before the barrier that ended the previous chunk's step 6,
        // and the next chunk reads it after the barrier below.
        if (w == kSW && c + 1 < n_chunks)
            step_values(buf ^ 1, pdt, (int)min((int64_t)kQ, p.L - t0 - kQ));
        __syncthreads();

        // ---- 5. this wave's channels: Y = M x + e^Λ C H, S = B^T (w x) -----
        f32x4 yd[TB], yo[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            yd[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            yo[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            const int tb = tile_tb(k), sb = tile_sb(k);
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
            split2(Hs[nb][0], Hs[nb][1], Hh[nb][0], Hl[nb][0]);
            split2(Hs[nb][2], Hs[nb][3], Hh[nb][1], Hl[nb][1]);
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
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

        // ---- 6. output tile to LDS, state update ------------------------------
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * g4 + i;
                sY[t * kYP + pcol] = fmaf(cEL[t], yo[tb][i], yd[tb][i]);
            }
        }
        const float decay = sDecay[buf];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Hs[nb][i] = fmaf(decay, Hs[nb][i], sa[nb][i]);
        }
        __syncthreads();
        // ---- 7. skip, gate and store: step xr, channels xc .. xc + kXPer - 1 --
        if (xr < nt) {
            uint16_t *yp = p.y + ((b * p.L + t0) * p.H + h) * kP + (xr * ts + xc);
#pragma unroll
            for (int k = 0; k < kXPer / 8; ++k) {
                const uint32_t xw[4] = {cX[k].x, cX[k].y, cX[k].z, cX[k].w};
                const uint32_t zw[4] = {cZ[k].x, cZ[k].y, cZ[k].z, cZ[k].w};
                uint32_t out[4];
                // the thread's 8 values as two 16-byte reads; threads with
                // xc >= 32 read their upper half first, so that each read's 8
                // lanes (one row) hit 32 different banks
                const float *yrow = sY + xr * kYP + xc + 8 * k;
                const int sw = (xc >> 5) & 1;
                const float4 fa = *reinterpret_cast<const float4 *>(yrow + 4 * sw);
                const float4 fb = *reinterpret_cast<const float4 *>(yrow + 4 * (sw ^ 1));
                const float4 lo = sw ? fb : fa, hi = sw ? fa : fb;
                const float yv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v0 = fmaf(Dv, __uint_as_float(xw[j] << 16), yv[2 * j]);
                    float v1 = fmaf(Dv, __uint_as_float(xw[j] & 0xffff0000u), yv[2 * j + 1]);
                    if (p.z) {
                        v0 *= silu_hw(__uint_as_float(zw[j] << 16));
                        v1 *= silu_hw(__uint_as_float(zw[j] & 0xffff0000u));
                    }
                    out[j] = cvt2(v0, v1);
                }
                *reinterpret_cast<uint4 *>(yp + 8 * k) = make_uint4(out[0], out[1], out[2], out[3]);
            }
        }
        // No barrier here: the next chunk's staging writes only B, C and x,
        // which nothing reads after the barrier above; Y is next written after
        // two more barriers, which every wave reaches only once its output is
        // stored.
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
    case 16: hipLaunchKernelGGL((ssd_fwd_kernel<16, ssd_chunk<16>()>), grid, block, 0, s, k); break;
    case 32: hipLaunchKernelGGL((ssd_fwd_kernel<32, ssd_chunk<32>()>), grid, block, 0, s, k); break;
    case 64: hipLaunchKernelGGL((ssd_fwd_kernel<64, ssd_chunk<64>()>), grid, block, 0, s, k); break;
    case 128: hipLaunchKernelGGL((ssd_fwd_kernel<128, ssd_chunk<128>()>), grid, block, 0, s, k); break;
    default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (a.ev_stop)
        (void)hipEventRecord(a.ev_stop, s);
    return e;
}

}  // namespace mamba
