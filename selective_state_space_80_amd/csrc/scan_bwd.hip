// Backward pass of the selective scan for gfx950: the gradients of
// J = sum(out * dout) (+ sum(h_last * dh_last)) with respect to x, dt, z, A, B,
// C, D, dt_bias and h0, with the forward states recomputed instead of stored
// ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式" §2.2:
// intermediate states are recomputed in the backward pass).
//
// Per channel and state n, with λ_t = dJ/dh_t and ν_t = Ā_t λ_t:
//   λ_t = C_t dy_t + ν_(t+1),   ν_L = dh_last,   dy_t = dout_t SiLU(z_t)
//   dx_t  = D dy_t + Σ_n λ_tn B̄coef_tn B_tn        (B̄coef = (e^(ΔA_n) - 1)/A_n)
//   dΔ_t  = Σ_n λ_tn Ā_tn (A_n h_(t-1),n + B_tn x_t),   ddt_t = dΔ_t σ(dt_t + bias)
//   dz_t  = dout_t (y_t + D x_t) SiLU'(z_t)
//   dA_n += λ_tn (Δ_t Ā_tn h_(t-1),n + Δ_t² ψ(Δ_t A_n) B_tn x_t)
//   dB_tn += λ_tn B̄coef_tn x_t,   dC_tn += dy_t h_tn   (summed over channels)
//   dD += dy_t x_t,   ddt_bias += ddt_t,   dh0 = ν_0
// The library runs it in four launches (see launch_selective_scan_bwd):
//   1. the forward scan, saving every 32-step chunk's start state;
//   2. the adjoint scan ν, in reverse time with the forward scan's machinery,
//      saving every chunk's incoming ν (from the future) and writing dh0;
//   3. this file's chunk kernel: per 64-channel tile and chunk, four lanes per
//      channel (one quarter of the 16 states each) recompute the chunk's
//      states four steps at a time from checkpoints, keeping each step's
//      decay and input coefficient, walk them backwards, and write dx, ddt,
//      dz and per-tile / per-chunk partial sums of dB, dC, dA, dD, ddt_bias;
//   4. a reduction of those partial sums in a fixed order (deterministic).
#include <cstddef>

#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

constexpr int kBT = 32;              // steps per chunk (the forward chunk grid)
constexpr int kSub = 4;              // steps whose states stay in registers at a time
constexpr int kNSub = kBT / kSub;    // sub-chunks per chunk, each from its own checkpoint
constexpr int kBThreads = 256;       // 64 channels x 4 lanes (4 states each)
constexpr int kCh = kBThreads / 4;   // channels per workgroup (one tile)
constexpr int kPad = kBT + 1;        // LDS row stride of the per-channel arrays
// row of sT: dB then dC of two steps (32 floats each) and two float4s of room
// for the odd channels' shift
constexpr int kTStride = 4 * kMaxN + 8;

// dβ/dA for β(A) = (e^(ΔA) - 1)/A, u = ΔA, e = e^u:  Δ² ψ(u) with
// ψ(u) = (u e^u - e^u + 1)/u² = Σ_m (m+1) u^m / (m+2)!, by its series through
// u^4 for |u| < 1/8 (truncation below 1e-7 relative); otherwise the same
// quantity as (Δ e - β)/A (β = (e - 1)/A), whose cancellation there costs at
// most a factor 2/|u| <= 16 in relative rounding error.
__device__ __forceinline__ float dbeta_dA(float delta, float del2, float u, float e, float beta,
                                          float rcpa)
{
    float s = 5.f / 720.f;  // (m+1)/(m+2)! for m = 4 .. 0
    s = fmaf(s, u, 4.f / 120.f);
    s = fmaf(s, u, 3.f / 24.f);
    s = fmaf(s, u, 2.f / 6.f);
    s = fmaf(s, u, 0.5f);
    const float closed = fmaf(delta, e, -beta) * rcpa;
    return fabsf(u) < 0.125f ? del2 * s : closed;
}

struct BwdArgs {
    const void *x, *dt, *z, *dout, *Bm, *Cm;
    const float *dt_bias, *A, *Dskip;
    const float *hsave, *nusave;  // [groups][n_cslots][16][64]
    void *dx, *ddt, *dz;          // [B, D, L] of the I/O type (dz NULL iff z NULL)
    float *dBp, *dCp;             // [n_dtiles][B][L][16] partial sums over 64 channels
    float *dAp;                   // [B * n_chunks][D][16]
    float *dDp, *dbp;             // [B * n_chunks][D]
    const uint32_t *tiles;        // [n_dtiles] class of each tile's A (the scan's table)
    int64_t B, D, L, n_dtiles, n_chunks, n_cslots;
    int N;
};

// LDS of the chunk kernel.  It stays under a third of the CU's 160 KB and the
// registers under 168, so that three workgroups (three waves per SIMD) share a
// CU.
struct BwdSmem {
    float sB[kBT][kMaxN];
    float sC[kBT][kMaxN];
    // per channel and step: Δ, x, dy; once a step is done its slots hold dΔ
    // (sDel, summed over the channel's states), dx (sX) and y + D x (sDY)
    float sDel[kCh][kPad], sX[kCh][kPad], sDY[kCh][kPad];
    // dB, dC of two steps per wave, channel-major, summed over the wave's 16
    // channels by reading them back transposed; the wave sums of a sub-chunk go
    // to sRed (two buffers: sub-chunks alternate).  A row is 18 float4s, so
    // consecutive channels start 2 float4s (8 banks) apart; odd channels store
    // 2 float4s further on, so that the 8 lanes of each 16-byte-store cycle (two
    // channels x four quarters) hit 32 different banks.
    float sT[kBThreads / 64][16][kTStride];
    float sRed[2][kBThreads / 64][kSub][2 * kMaxN];
};
static_assert(offsetof(BwdSmem, sC) % 16 == 0 && offsetof(BwdSmem, sT) % 16 == 0,
              "rows read and written as float4");
// 54016 bytes (sT rows of 20 float4s) measured at two workgroups per CU
static_assert(sizeof(BwdSmem) <= 52 * 1024, "three workgroups per CU");

// The whole chunk computation for one class of A (STRUCT: the structured form,
// whose recompute takes the decays of a step's states as powers of one
// exponential).
template <bool BF16, bool STRUCT>
__device__ __forceinline__ void bwd_chunk(const BwdArgs &p, BwdSmem &sm)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    auto &sB = sm.sB;
    auto &sC = sm.sC;
    auto &sDel = sm.sDel;
    auto &sX = sm.sX;
    auto &sDY = sm.sDY;
    auto &sT = sm.sT;
    auto &sRed = sm.sRed;

    const int64_t wg = blockIdx.x;
    const int64_t c = wg % p.n_chunks;         // chunk
    const int64_t g = wg / p.n_chunks;         // group = b * n_dtiles + tile
    const int64_t b = g / p.n_dtiles, tile = g - b * p.n_dtiles;
    const int tid = threadIdx.x;
    const int ch = tid >> 2, q = tid & 3, wave = tid >> 6;
    const int64_t d = tile * kCh + ch;
    const bool active = d < p.D;
    const int64_t dc = active ? d : p.D - 1;
    const int64_t t0 = c * kBT;
    const int nt = (int)min((int64_t)kBT, p.L - t0);
    const T *Bb = reinterpret_cast<const T *>(p.Bm) + b * p.L * p.N;
    const T *Cb = reinterpret_cast<const T *>(p.Cm) + b * p.L * p.N;

    // ---- stage B, C rows and the per-channel step values ------------------
    // Every load below is issued before any is used, with no branch around
    // them: out-of-range elements read index 0 and are masked to 0 (a branch
    // around a load makes the compiler wait for all earlier loads at the join).
    // Steps past L and channels past D are identity steps with zero input and
    // zero output gradient: they add nothing to dB, dC.
    {
        constexpr int kBC = kBT * kMaxN / kBThreads;  // B, C values per thread
        constexpr int kPS = kCh * kBT / kBThreads;    // per-channel elements per thread
        static_assert(kBThreads % kBT == 0, "one step per thread in the staging");
        float bq[kBC], cq[kBC];
        bool okbc[kBC];
#pragma unroll
        for (int k = 0; k < kBC; ++k) {
            const int e = tid + k * kBThreads, r = e / kMaxN, n = e % kMaxN;
            okbc[k] = r < nt && n < p.N;
            const int64_t o = okbc[k] ? (t0 + r) * p.N + n : 0;
            bq[k] = E::load(Bb + o);
            cq[k] = E::load(Cb + o);
        }
        const int r = tid % kBT;  // this thread's step; channels tid/kBT + k kBThreads/kBT
        const T *dtp = reinterpret_cast<const T *>(p.dt), *xp = reinterpret_cast<const T *>(p.x);
        const T *gp = reinterpret_cast<const T *>(p.dout);
        const T *zp = reinterpret_cast<const T *>(p.z ? p.z : p.dout);
        const float *biasp = p.dt_bias ? p.dt_bias : p.A;  // A has at least D entries
        float dtv[kPS], xq[kPS], gq[kPS], zq[kPS], bq2[kPS];
        bool ok[kPS];
#pragma unroll
        for (int k = 0; k < kPS; ++k) {
            const int cc = tid / kBT + k * (kBThreads / kBT);
            const int64_t dd = tile * kCh + cc;
            ok[k] = r < nt && dd < p.D;
            const int64_t i = ok[k] ? (b * p.D + dd) * p.L + t0 + r : 0;
            dtv[k] = E::load(dtp + i);
            xq[k] = E::load(xp + i);
            gq[k] = E::load(gp + i);
            zq[k] = E::load(zp + i);
            bq2[k] = biasp[ok[k] ? dd : 0];
        }
#pragma unroll
        for (int k = 0; k < kBC; ++k) {
            const int e = tid + k * kBThreads;
            sB[e / kMaxN][e % kMaxN] = okbc[k] ? bq[k] : 0.f;
            sC[e / kMaxN][e % kMaxN] = okbc[k] ? cq[k] : 0.f;
        }
        const float bias_on = p.dt_bias ? 1.f : 0.f;
#pragma unroll
        for (int k = 0; k < kPS; ++k) {
            const int cc = tid / kBT + k * (kBThreads / kBT);
            const float v = dtv[k] + bias_on * bq2[k];
            const float gate = p.z ? silu_hw(zq[k]) : 1.f;
            sDel[cc][r] = ok[k] ? softplus_log2(v * kLog2e) * kLn2 : 0.f;
            sX[cc][r] = ok[k] ? xq[k] : 0.f;
            sDY[cc][r] = ok[k] ? gq[k] * gate : 0.f;
        }
    }
    __syncthreads();

    // ---- per-lane constants: states n = 4q + i of channel dc --------------
    // (loads first and unconditional, as above; dc is always a valid channel)
    float a[4], rcpa[4], nu[4], dAacc[4];
    float ck[kNSub][4];  // state at the start of each sub-chunk
    float araw[4], hraw[4], nraw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = 4 * q + i;
        const int64_t cs = ((g * p.n_cslots + c) * kMaxN + n) * 64 + ch;
        araw[i] = p.A[dc * p.N + min(n, p.N - 1)];
        hraw[i] = p.hsave[cs];
        nraw[i] = p.nusave[cs];
    }
    const float a0raw = p.A[dc * p.N];
    const float Draw = (p.Dskip ? p.Dskip : p.A)[dc];
    // structured: A_0 of the channel (its states' decays are powers of e^(ΔA_0))
    const float a0 = STRUCT && active ? a0raw : -1.f;
    const float rcpa0 = hw_rcp(a0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool live = active && 4 * q + i < p.N;  // other states stay exactly zero
        a[i] = live ? araw[i] : 0.f;
        rcpa[i] = a[i] != 0.f ? hw_rcp(a[i]) : 0.f;
        ck[0][i] = live ? hraw[i] : 0.f;
        nu[i] = live ? nraw[i] : 0.f;
        dAacc[i] = 0.f;
    }
    const float Dd = p.Dskip ? Draw : 0.f;
    float dDacc = 0.f;

    // one forward step of the lane's four states; e_n = exp(Δ A_n) and the
    // input coefficient β_n = (e_n - 1)/A_n are returned for the caller.
    // Structured A (A_n = (n+1) A_0): the lane's first state n = 4q as in the
    // general form, then e_n - 1 = e (e_(n-1) - 1) + (e - 1) with e = e^(ΔA_0)
    // for the next three, e - 1 from φ1's series near 0 (no cancellation), so
    // each β_n = (e_n - 1)/A_n keeps full relative accuracy.
    auto fwd = [&](int r, float (&h)[4], float (&ev)[4], float (&bv)[4]) {
        const float del = sDel[ch][r], xv = sX[ch][r];
        const float l = del * kLog2e;
        const float4 B4 = *reinterpret_cast<const float4 *>(&sB[r][4 * q]);
        const float Bv[4] = {B4.x, B4.y, B4.z, B4.w};
        if constexpr (STRUCT) {
            const float w0 = a0 * l;
            const float e1 = hw_exp2(w0);
            const float em0 = zoh_coef_w(w0, del, e1, rcpa0) * a0;  // e - 1
            const float wq = a[0] * l;
            ev[0] = hw_exp2(wq);
            bv[0] = zoh_coef_w(wq, del, ev[0], rcpa[0]);
            float em = bv[0] * a[0];  // e_n - 1 of the lane's first state
            h[0] = fmaf(ev[0], h[0], bv[0] * (Bv[0] * xv));
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                em = fmaf(e1, em, em0);
                ev[i] = em + 1.f;
                bv[i] = em * rcpa[i];
                h[i] = fmaf(ev[i], h[i], bv[i] * (Bv[i] * xv));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float w = a[i] * l;
                ev[i] = hw_exp2(w);
                bv[i] = zoh_coef_w(w, del, ev[i], rcpa[i]);
                h[i] = fmaf(ev[i], h[i], bv[i] * (Bv[i] * xv));
            }
        }
    };

    // one sub-chunk [r0, r0 + kSub): states, decays and input coefficients
    // from hstart kept in registers, then walked backwards
    auto sub_chunk = [&](int r0, const float (&hstart)[4], float (*red)[kSub][2 * kMaxN]) {
        float H[kSub][4], Ev[kSub][4], Bt[kSub][4];
        {
            float h[4] = {hstart[0], hstart[1], hstart[2], hstart[3]};
#pragma unroll
            for (int j = 0; j < kSub; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                fwd(r0 + j, h, Ev[j], Bt[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    H[j][i] = h[i];
            }
        }
#pragma unroll
        for (int j = kSub - 1; j >= 0; --j) {
            __builtin_amdgcn_sched_barrier(0);
            const int r = r0 + j;
            const float del = sDel[ch][r], xv = sX[ch][r], dy = sDY[ch][r];
            const float4 B4 = *reinterpret_cast<const float4 *>(&sB[r][4 * q]);
            const float4 C4 = *reinterpret_cast<const float4 *>(&sC[r][4 * q]);
            const float Bv[4] = {B4.x, B4.y, B4.z, B4.w}, Cv[4] = {C4.x, C4.y, C4.z, C4.w};
            const float del2 = del * del;
            float dxp = 0.f, ddel = 0.f, yp = 0.f, dBv[4], dCv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float hp = j ? H[j - 1][i] : hstart[i];
                const float ht = H[j][i];
                const float e = Ev[j][i], beta = Bt[j][i];
                const float u = a[i] * del;
                const float lam = fmaf(Cv[i], dy, nu[i]);
                const float bx = Bv[i] * xv;
                const float lb = lam * beta;
                const float le = lam * e;
                dCv[i] = dy * ht;
                dBv[i] = lb * xv;
                dxp = fmaf(lb, Bv[i], dxp);
                ddel = fmaf(le, fmaf(a[i], hp, bx), ddel);
                dAacc[i] = fmaf(del * le, hp, fmaf(lam * bx, dbeta_dA(del, del2, u, e, beta, rcpa[i]),
                                                   dAacc[i]));
                yp = fmaf(Cv[i], ht, yp);
                nu[i] = le;
            }
            dxp = quad_sum(dxp);
            ddel = quad_sum(ddel);
            yp = quad_sum(yp);
            // every lane of the quad holds the sums; lane 0 stores them (all
            // four storing the same words measured 2% slower).  Δ, x and dy of
            // step r are not read again.
            dDacc = fmaf(dy, xv, dDacc);     // padded steps have dy = x = 0
            if (q == 0) {
                sDel[ch][r] = ddel;              // dΔ (times σ at the output)
                sX[ch][r] = fmaf(Dd, dy, dxp);   // dx
                sDY[ch][r] = fmaf(Dd, xv, yp);   // y + D x, for dz
            }
            // dB, dC: sums over the wave's 16 channels.  Two steps at a time: the
            // lanes store their values channel-major, then lane l adds up the
            // 16 channels of entry l (step j + l/32, value l%32) in order.
            const int s2 = j & 1;
            const int wc = (tid & 63) >> 2;  // the lane's channel within the wave
            float4 *row = reinterpret_cast<float4 *>(&sT[wave][wc][(wc & 1) * 8 + s2 * 2 * kMaxN]);
            row[q] = make_float4(dBv[0], dBv[1], dBv[2], dBv[3]);
            row[4 + q] = make_float4(dCv[0], dCv[1], dCv[2], dCv[3]);
            if (s2 == 0) {
                __builtin_amdgcn_wave_barrier();
                const int l = tid & 63, so = l >> 5, kn = l & 31;
                float acc = 0.f;
#pragma unroll
                for (int cw = 0; cw < 16; ++cw)
                    acc += sT[wave][cw][(cw & 1) * 8 + l];
                red[wave][j + so][kn] = acc;
                __builtin_amdgcn_wave_barrier();
            }
            // keep the accumulators' chains in their steps (otherwise the
            // compiler sinks them to the end and every operand stays live)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __asm__ volatile("" : "+v"(dAacc[i]), "+v"(nu[i]));
        }
    };

    // Checkpoints: the states at the starts of the sub-chunks, from one
    // forward pass over all but the last sub-chunk.  Then the sub-chunks from
    // the last to the first, each recomputed from its checkpoint; the adjoint
    // carries on from one to the next.  A loop, not eight copies, so that
    // nothing of one sub-chunk stays live into the next.
    {
        float h[4] = {ck[0][0], ck[0][1], ck[0][2], ck[0][3]}, ev[4], bv[4];
#pragma unroll
        for (int j = 0; j < kBT - kSub; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            fwd(j, h, ev, bv);
            if ((j + 1) % kSub == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ck[(j + 1) / kSub][i] = h[i];
            }
        }
    }
#pragma unroll 1
    for (int k = kNSub - 1; k >= 0; --k) {
        float hst[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = ck[0][i];
#pragma unroll
            for (int m = 1; m < kNSub; ++m)
                v = k == m ? ck[m][i] : v;
            hst[i] = v;
        }
        const int buf = k & 1;
        sub_chunk(k * kSub, hst, sRed[buf]);
        // every wave has its sums of the sub-chunk's steps in sRed[buf]: add
        // them in wave order and store the tile's partial dB, dC rows.  The
        // buffer is written again two sub-chunks later, after the next
        // barrier, which these threads reach only once they are done here.
        __syncthreads();
        if (tid < kSub * 2 * kMaxN) {
            const int ss = tid / (2 * kMaxN), kn = tid % (2 * kMaxN);
            const int r = k * kSub + ss;
            if (r < nt) {
                float v = sRed[buf][0][ss][kn];
#pragma unroll
                for (int wv = 1; wv < kBThreads / 64; ++wv)
                    v += sRed[buf][wv][ss][kn];
                const int64_t o = ((tile * p.B + b) * p.L + t0 + r) * kMaxN + (kn % kMaxN);
                (kn < kMaxN ? p.dBp : p.dCp)[o] = v;
            }
        }
    }

    // ---- outputs ----------------------------------------------------------
    // ddt = dΔ σ(dt + bias) (dΔ/d(dt) = σ), formed here once per element; it
    // replaces dΔ in sDel for the ddt_bias sums below.  As in the staging, the
    // loads of a group of elements are issued first and unconditionally (index
    // 0 for elements out of range) and only the stores are conditional; two
    // groups of four, so that the registers stay within budget.
    {
        constexpr int kPS = kCh * kBT / kBThreads;
        constexpr int kGrp = kPS / 2;
        const int r = tid % kBT;
        const T *dtp = reinterpret_cast<const T *>(p.dt);
        const T *zp = reinterpret_cast<const T *>(p.z ? p.z : p.dout);
        const T *gp = reinterpret_cast<const T *>(p.dout);
        const float *biasp = p.dt_bias ? p.dt_bias : p.A;
        const float bias_on = p.dt_bias ? 1.f : 0.f;
#pragma unroll 1
        for (int k0 = 0; k0 < kPS; k0 += kGrp) {
            float dtv[kGrp], zq[kGrp], gq[kGrp], bq[kGrp];
#pragma unroll
            for (int k = 0; k < kGrp; ++k) {
                const int cc = tid / kBT + (k0 + k) * (kBThreads / kBT);
                const int64_t dd = tile * kCh + cc;
                const bool ok = dd < p.D && r < nt;
                const int64_t i = ok ? (b * p.D + dd) * p.L + t0 + r : 0;
                dtv[k] = E::load(dtp + i);
                zq[k] = E::load(zp + i);
                gq[k] = E::load(gp + i);
                bq[k] = biasp[ok ? dd : 0];
            }
#pragma unroll
            for (int k = 0; k < kGrp; ++k) {
                const int cc = tid / kBT + (k0 + k) * (kBThreads / kBT);
                const int64_t dd = tile * kCh + cc;
                const float v = dtv[k] + bias_on * bq[k];
                const float ddt = sDel[cc][r] * hw_rcp(1.f + hw_exp2(-v * kLog2e));
                // dz = dout (y + D x) SiLU'(z), SiLU'(z) = σ(z)(1 + z(1 - σ(z)))
                const float sz = hw_rcp(1.f + hw_exp2(-zq[k] * kLog2e));
                const float dzv = gq[k] * sDY[cc][r] * sz * fmaf(zq[k], 1.f - sz, 1.f);
                if (dd < p.D && r < nt) {
                    const int64_t i = (b * p.D + dd) * p.L + t0 + r;
                    sDel[cc][r] = ddt;
                    E::store(reinterpret_cast<T *>(p.dx) + i, sX[cc][r]);
                    E::store(reinterpret_cast<T *>(p.ddt) + i, ddt);
                    if (p.dz)
                        E::store(reinterpret_cast<T *>(p.dz) + i, dzv);
                }
            }
        }
    }
    __syncthreads();
    if (active) {
        const int64_t bc = b * p.n_chunks + c;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p.dAp[(bc * p.D + d) * kMaxN + 4 * q + i] = dAacc[i];
        if (q == 0) {
            // the chunk's ddt_bias share: its ddt values in step order
            float db = 0.f;
            for (int r = 0; r < nt; ++r)
                db += sDel[ch][r];
            p.dDp[bc * p.D + d] = dDacc;
            p.dbp[bc * p.D + d] = db;
        }
    }
}

template <bool BF16>
__global__ void __launch_bounds__(kBThreads, 3) scan_bwd_chunk_kernel(BwdArgs p)
{
    __shared__ __align__(16) BwdSmem sm;
    const int64_t tile = (blockIdx.x / p.n_chunks) % p.n_dtiles;
    const uint32_t path = __builtin_amdgcn_readfirstlane(p.tiles[tile]);
    if (path == kPathStructured)
        bwd_chunk<BF16, true>(p, sm);
    else
        bwd_chunk<BF16, false>(p, sm);
}

// Fixed-order column sums of a [rows][cols] partial array:
//   out[o * n_out + n] = Σ_r in[r][o * inner + n]   for n < n_out.
// A workgroup takes 256/RG columns; RG row groups per column each add every
// RG-th row with four interleaved accumulators, then one thread per column
// adds the groups in order.  The result depends on the shape only.
template <int RG>
__global__ void __launch_bounds__(256) colsum_kernel(const float *__restrict__ in,
                                                     float *__restrict__ out, int64_t rows,
                                                     int64_t cols, int inner, int n_out)
{
    constexpr int kCols = 256 / RG;
    __shared__ float part[RG][kCols];
    const int cg = threadIdx.x % kCols, rg = threadIdx.x / kCols;
    const int64_t col = (int64_t)blockIdx.x * kCols + cg;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (col < cols) {
        int64_t r = rg;
        for (; r + 3 * RG < rows; r += 4 * RG) {
            s0 += in[r * cols + col];
            s1 += in[(r + RG) * cols + col];
            s2 += in[(r + 2 * RG) * cols + col];
            s3 += in[(r + 3 * RG) * cols + col];
        }
        for (; r < rows; r += RG)
            s0 += in[r * cols + col];
    }
    part[rg][cg] = (s0 + s1) + (s2 + s3);
    __syncthreads();
    if (rg == 0 && col < cols) {
        float t = part[0][cg];
#pragma unroll
        for (int k = 1; k < RG; ++k)
            t += part[k][cg];
        const int64_t o = col / inner;
        const int n = (int)(col - o * inner);
        if (n < n_out)
            out[o * n_out + n] = t;
    }
}

hipError_t colsum(const float *in, float *out, int64_t rows, int64_t cols, int inner, int n_out,
                  hipStream_t s)
{
    if (!out || cols == 0)
        return hipSuccess;
    if (rows >= 64) {  // long sums: 16 row groups of 16 columns
        hipLaunchKernelGGL(colsum_kernel<16>, dim3((unsigned)((cols + 15) / 16)), dim3(256), 0,
                           s, in, out, rows, cols, inner, n_out);
    } else {
        hipLaunchKernelGGL(colsum_kernel<4>, dim3((unsigned)((cols + 63) / 64)), dim3(256), 0,
                           s, in, out, rows, cols, inner, n_out);
    }
    return hipGetLastError();
}

// Nothing to scan (L = 0 or B = 0): the parameter gradients are empty sums
// and dh0 = dh_last.
__global__ void __launch_bounds__(256) scan_bwd_empty_kernel(float *dA, float *dD,
                                                             float *ddt_bias, float *dh0,
                                                             const float *dh_last, int64_t n_a,
                                                             int64_t D, int64_t n_h)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_a)
        dA[i] = 0.f;
    if (i < D) {
        if (dD)
            dD[i] = 0.f;
        if (ddt_bias)
            ddt_bias[i] = 0.f;
    }
    if (dh0 && i < n_h)
        dh0[i] = dh_last ? dh_last[i] : 0.f;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

BwdWsLayout scan_bwd_ws_layout(int64_t B, int64_t D, int64_t L)
{
    BwdWsLayout w;
    w.scan = scan_ws_layout(B, D, L);
    const int64_t n_cslots = w.scan.n_seg * kWavesPerSeg;
    const int64_t n_chunks = (L + kBT - 1) / kBT;
    size_t off = align256(w.scan.total);
    w.off_hsave = off;
    off = align256(off + (size_t)w.scan.groups * n_cslots * kMaxN * 64 * 4);
    w.off_nusave = off;
    off = align256(off + (size_t)w.scan.groups * n_cslots * kMaxN * 64 * 4);
    w.off_dBp = off;
    off = align256(off + (size_t)w.scan.n_dtiles * B * L * kMaxN * 4);
    w.off_dCp = off;
    off = align256(off + (size_t)w.scan.n_dtiles * B * L * kMaxN * 4);
    w.off_dAp = off;
    off = align256(off + (size_t)B * n_chunks * D * kMaxN * 4);
    w.off_dDp = off;
    off = align256(off + (size_t)B * n_chunks * D * 4);
    w.off_dbp = off;
    off = align256(off + (size_t)B * n_chunks * D * 4);
    w.total = off;
    return w;
}

hipError_t launch_selective_scan_bwd(const BwdArgsHost &a, hipStream_t s)
{
    if (a.D == 0)
        return hipSuccess;
    if (a.L == 0 || a.B == 0) {
        const int64_t n_a = a.D * a.N, n_h = a.B * a.D * a.N;
        const int64_t n = max(n_a, n_h);
        hipLaunchKernelGGL(scan_bwd_empty_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, s, a.dA, a.dD, a.ddt_bias, a.dh0, a.dh_last, n_a, a.D, n_h);
        return hipGetLastError();
    }
    const BwdWsLayout w = scan_bwd_ws_layout(a.B, a.D, a.L);
    unsigned char *ws = a.ws;
    float *hsave = reinterpret_cast<float *>(ws + w.off_hsave);
    float *nusave = reinterpret_cast<float *>(ws + w.off_nusave);
    // 1. forward scan, saving chunk start states (no output)
    ScanArgs f;
    f.x = a.x;
    f.dt = a.dt;
    f.Bm = a.Bm;
    f.Cm = a.Cm;
    f.z = nullptr;
    f.dt_bias = a.dt_bias;
    f.A = a.A;
    f.Dskip = nullptr;
    f.h0 = a.h0;
    f.y = nullptr;
    f.h_last = nullptr;
    f.ws = ws;
    f.lay = w.scan;
    f.B = a.B;
    f.D = a.D;
    f.L = a.L;
    f.N = a.N;
    f.bf16 = a.bf16;
    f.conv_K = 0;
    f.conv_w = f.conv_b = nullptr;
    f.conv_state_in = nullptr;
    f.conv_state_out = nullptr;
    f.reverse = false;
    f.accumulate = false;
    f.adjoint = false;
    f.chunk_states = hsave;
    f.keep_error = false;
    f.spin_limit = a.spin_limit;
    f.ev_start = f.ev_stop = nullptr;
    hipError_t e = launch_selective_scan(f, s);
    if (e != hipSuccess)
        return e;
    // 2. adjoint scan in reverse time: x = dout, incoming state dh_last,
    //    final state dh0, chunk incoming adjoints saved
    ScanArgs r = f;
    r.x = a.dout;
    r.z = a.z;
    r.h0 = a.dh_last;
    r.h_last = a.dh0;
    r.reverse = true;
    r.adjoint = true;
    r.chunk_states = nusave;
    r.keep_error = true;  // the forward scan's timeout, if any, stays reported
    e = launch_selective_scan(r, s);
    if (e != hipSuccess)
        return e;
    // 3. chunk gradients
    BwdArgs k;
    k.x = a.x;
    k.dt = a.dt;
    k.z = a.z;
    k.dout = a.dout;
    k.Bm = a.Bm;
    k.Cm = a.Cm;
    k.dt_bias = a.dt_bias;
    k.A = a.A;
    k.Dskip = a.Dskip;
    k.hsave = hsave;
    k.nusave = nusave;
    k.dx = a.dx;
    k.ddt = a.ddt;
    k.dz = a.dz;
    k.dBp = reinterpret_cast<float *>(ws + w.off_dBp);
    k.dCp = reinterpret_cast<float *>(ws + w.off_dCp);
    k.dAp = reinterpret_cast<float *>(ws + w.off_dAp);
    k.dDp = reinterpret_cast<float *>(ws + w.off_dDp);
    k.dbp = reinterpret_cast<float *>(ws + w.off_dbp);
    k.tiles = reinterpret_cast<const uint32_t *>(ws + w.scan.off_tiles);
    k.B = a.B;
    k.D = a.D;
    k.L = a.L;
    k.n_dtiles = w.scan.n_dtiles;
    k.n_chunks = (a.L + kBT - 1) / kBT;
    k.n_cslots = w.scan.n_seg * kWavesPerSeg;
    k.N = a.N;
    const dim3 grid((unsigned)(w.scan.groups * k.n_chunks));
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, s);
    if (a.bf16)
        hipLaunchKernelGGL(scan_bwd_chunk_kernel<true>, grid, dim3(kBThreads), 0, s, k);
    else
        hipLaunchKernelGGL(scan_bwd_chunk_kernel<false>, grid, dim3(kBThreads), 0, s, k);
    e = hipGetLastError();
    if (a.ev_stop)
        (void)hipEventRecord(a.ev_stop, s);
    if (e != hipSuccess)
        return e;
    // 4. reductions: dB, dC over tiles; dA, dD, ddt_bias over (b, chunk)
    const int64_t rows_t = w.scan.n_dtiles, rows_c = a.B * k.n_chunks;
    const int64_t cols_bc = a.B * a.L * kMaxN;
    if ((e = colsum(k.dBp, a.dB, rows_t, cols_bc, kMaxN, a.N, s)) != hipSuccess ||
        (e = colsum(k.dCp, a.dC, rows_t, cols_bc, kMaxN, a.N, s)) != hipSuccess ||
        (e = colsum(k.dAp, a.dA, rows_c, a.D * kMaxN, kMaxN, a.N, s)) != hipSuccess ||
        (e = colsum(k.dDp, a.dD, rows_c, a.D, 1, 1, s)) != hipSuccess ||
        (e = colsum(k.dbp, a.ddt_bias, rows_c, a.D, 1, 1, s)) != hipSuccess)
        return e;
    return hipGetLastError();
}

}  // namespace mamba
