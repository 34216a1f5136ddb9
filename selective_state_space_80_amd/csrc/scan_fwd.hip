// Fused selective-scan forward for gfx950 (MI355X).
//
// What is computed, per channel (b, d) and time step t (Mamba's selective SSM):
//   Δ_t = softplus(dt_t + dt_bias_d)                       ["Mamba架构与SSM模型：
//   Ā_t = exp(Δ_t A_dn),  B̄_t = (Δ_t A)^-1 (exp(Δ_t A)-1) Δ_t B_tn   高效序列建模技术解析" §2.1-2.2]
//   h_tn = Ā_t h_(t-1)n + B̄_t x_t,  y_t = sum_n C_tn h_tn + D_d x_t
//                                        ["Mamba状态空间模型深度解析…" §2.1]
//   out_t = y_t * SiLU(z_t)              [same page, §3.1 gated block]
//
// Mapping onto CDNA4
//   * lane = channel.  A wave owns 64 consecutive channels of one batch row and
//     keeps their N <= 16 fp32 states in VGPRs while it walks time.  B_t and C_t
//     are the same for all 64 lanes, so they are wave-uniform scalar loads
//     (SGPR operands), not per-lane traffic.
//   * Work is cut into segments of kSegT = 4 x 32 steps.  Each of the 4 waves of
//     a workgroup scans one 32-step chunk from a zero state, keeping its 32
//     partial outputs and decay factors in registers (fully unrolled loop).
//   * The end state of a chunk is an affine map h -> P h + S of its start state
//     (the block-wise scan with a prefix state handed to later blocks,
//     "Mamba: Linear-Time Sequence Modeling with Selective SSMs", selective scan
//     section).  Chunk maps are combined in LDS inside the workgroup.  Across
//     workgroups every segment publishes its map (an aggregate record) in the
//     workspace; segments are grouped 16 to a superblock, and the last segment
//     of a superblock also publishes the state at its end (an inclusive
//     record).  A segment's start state is the previous superblock's inclusive
//     state with the aggregates of the earlier segments of its own superblock
//     folded on top, in a fixed order, by the 4 waves in parallel.  The
//     association order therefore never depends on scheduling (results are
//     bit-for-bit repeatable), and the only serial chain is one hop per
//     superblock.  Segment ids come from an atomic ticket, so every segment a
//     wave waits for has already started: no deadlock whatever the dispatch
//     order.
//   * Once a chunk knows its true start state h_in, each kept output gets the
//     missing term sum_n C_tn * (prod_(s<=t) Ā_sn) * h_in,n added, then the
//     gate, then one store.  Every input element is read once, y written once.
//
// Two arithmetic paths, chosen per 64-channel tile by the prep kernel:
//   structured  A_dn = (n+1) A_d0 exactly with A_d0 < 0 (the S4D-real form).
//               Then exp(Δ A_dn) = e^(n+1) with e = exp(Δ A_d0): one exp per
//               element, powers by multiplication.  The state is kept scaled,
//               ĥ_n = A_dn h_n, which turns the ZOH update into
//               ĥ <- e_n (ĥ + B_n x) - B_n x   (exact algebra of
//               h <- e_n h + (e_n - 1)/A_n B_n x), so no division per state; the
//               readout uses C_n/(n+1) prepared once per (b, t) and 1/A_d0 per
//               channel.  5 VALU operations per state and step.
//   general     any A: per state exp and an accurate expm1 for B̄ (expm1f / A_n,
//               with the A_n = 0 limit Δ).  Slower, exact form.
#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

struct WsHeader {
    uint32_t ticket;
    uint32_t error;
    uint32_t pad[62];
};

constexpr uint32_t kFlagAgg = 1u;
constexpr uint32_t kFlagIncl = 2u;
constexpr uint32_t kPathStructured = 0u;
constexpr uint32_t kPathGeneral = 1u;
constexpr uint32_t kErrSpinTimeout = 1u;
constexpr int kSpinLimit = 1 << 22;
constexpr int64_t kSuperSeg = 16;  // segments per superblock of the carry

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Prep kernel: clears the ticket and the per-segment flags, converts B and C
// to fp32 rows [B | C/(n+1)] of exactly 128 bytes plus a separate array of C
// (16 entries each, zero past N; zero rows pad
// each batch row to a whole number of segments), and decides
// per 64-channel tile whether A has the structured form.
template <bool BF16>
__global__ void __launch_bounds__(256) scan_prep_kernel(
    const void *__restrict__ Bm_, const void *__restrict__ Cm_, const float *__restrict__ A,
    unsigned char *__restrict__ ws, ScanWsLayout lay, int64_t D, int64_t L, int N,
    int64_t n_zero, int64_t n_bc, int64_t classify_base)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_zero) {
        if (i == 0) {
            WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + lay.off_header);
            hdr->ticket = 0u;
            hdr->error = 0u;
        }
        if (i < lay.n_items)
            reinterpret_cast<uint32_t *>(ws + lay.off_flags)[i] = 0u;
        return;
    }
    if (i < n_zero + n_bc) {
        const int64_t k = i - n_zero;
        const int64_t row = k / kMaxN;  // b * Lpad + t
        const int n = (int)(k % kMaxN);
        const int64_t Lpad = lay.n_seg * kSegT;
        const int64_t b = row / Lpad, t = row - b * Lpad;
        float bv = 0.f, cv = 0.f;
        if (n < N && t < L) {
            bv = E::load(reinterpret_cast<const T *>(Bm_) + (b * L + t) * N + n);
            cv = E::load(reinterpret_cast<const T *>(Cm_) + (b * L + t) * N + n);
        }
        float *bc = reinterpret_cast<float *>(ws + lay.off_bc) + row * kBCStride;
        bc[n] = bv;
        bc[kMaxN + n] = cv / (float)(n + 1);
        reinterpret_cast<float *>(ws + lay.off_craw)[row * kMaxN + n] = cv;
        return;
    }
    const int64_t c = i - classify_base;  // classify region starts on a wave boundary
    if (c < 0 || c >= lay.n_dtiles * kWave)
        return;
    const int64_t d = c;
    bool ok = true;
    if (d < D) {
        const float a0 = A[d * N];
        ok = (a0 < -1e-30f) && (a0 > -1e30f);
        for (int n = 1; n < N; ++n)
            ok = ok && (A[d * N + n] == (float)(n + 1) * a0);
    }
    const uint64_t bad = __ballot(!ok);
    if ((threadIdx.x & (kWave - 1)) == 0)
        reinterpret_cast<uint32_t *>(ws + lay.off_tiles)[c / kWave] =
            bad ? kPathGeneral : kPathStructured;
}

// ---------------------------------------------------------------------------
// Per-lane chunk I/O: 32 consecutive time steps of one row.  `vec` means the
// chunk is full and the row is 16-byte aligned, so 128-bit loads are used.
// Steps at or past L are filled with `pad` and never stored: padding x with 0
// and dt with -inf makes such a step an exact identity of the recurrence
// (step 0, decay 1, no input), so the step loops need no per-step branches.
template <bool BF16>
__device__ __forceinline__ void load_chunk(const void *base, int64_t off, int nt, bool vec,
                                           float (&v)[kChunkT], float pad = 0.f)
{
    if constexpr (!BF16) {
        const float *p = reinterpret_cast<const float *>(base) + off;
        if (vec) {
            const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 4; ++i) {
                const float4 a = q[i];
                v[4 * i + 0] = a.x;
                v[4 * i + 1] = a.y;
                v[4 * i + 2] = a.z;
                v[4 * i + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kChunkT; ++i)
                v[i] = (i < nt) ? p[i] : pad;
        }
    } else {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + off;
        if (vec) {
            const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 8; ++i) {
                const uint4 a = q[i];
                const uint32_t w4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[8 * i + 2 * k + 0] = __uint_as_float(w4[k] << 16);
                    v[8 * i + 2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kChunkT; ++i)
                v[i] = (i < nt) ? bf16_bits_to_f32(p[i]) : pad;
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void store_chunk(void *base, int64_t off, int nt, bool vec,
                                            const float (&v)[kChunkT])
{
    if constexpr (!BF16) {
        float *p = reinterpret_cast<float *>(base) + off;
        if (vec) {
            float4 *q = reinterpret_cast<float4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 4; ++i)
                q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        } else {
#pragma unroll
            for (int i = 0; i < kChunkT; ++i)
                if (i < nt)
                    p[i] = v[i];
        }
    } else {
        uint16_t *p = reinterpret_cast<uint16_t *>(base) + off;
        if (vec) {
            uint4 *q = reinterpret_cast<uint4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 8; ++i) {
                uint32_t w4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w4[k] = f32_to_bf16_bits(v[8 * i + 2 * k]) |
                            (f32_to_bf16_bits(v[8 * i + 2 * k + 1]) << 16);
                q[i] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kChunkT; ++i)
                if (i < nt)
                    p[i] = (uint16_t)f32_to_bf16_bits(v[i]);
        }
    }
}

// Carry records between workgroups.  Every record word and every flag is
// accessed with agent-scope relaxed atomics, which are coherent across the
// XCDs' L2 caches without whole-cache write-back or invalidation.  A writer
// waits until all of its record stores have completed (vmcnt = 0) before it
// stores the flag; a reader loads record words only after it has seen the
// flag, so it reads this call's values.
__device__ __forceinline__ uint32_t load_flag(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_rec(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_rec(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish_flag(uint32_t *p, uint32_t v, int lane)
{
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ScanKArgs {
    const void *x, *dt, *z;
    void *y;
    const float *dt_bias, *A, *Dskip, *h0;
    float *h_last;
    unsigned char *ws;
    ScanWsLayout lay;
    int64_t B, D, L;
    int N;
    int vec;  // rows of x, dt, z, y are 16-byte aligned for vector access
};

// Decay factor P_n of an aggregate whose summary is f:
//   structured: f = prod e over the chunk, P_n = f^(n+1)
//   general:    f = sum over the chunk of Δ/ln2, P_n = 2^(A_n f)   (A_n = 0 -> 1)
template <bool STRUCT>
__device__ __forceinline__ void decay_factors(float f, const float (&Ar)[kMaxN],
                                              float (&P)[kMaxN])
{
    if constexpr (STRUCT) {
        float p = f;
#pragma unroll
        for (int n = 0; n < kMaxN; ++n) {
            P[n] = p;
            p *= f;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            P[n] = (Ar[n] == 0.f) ? 1.f : hw_exp2(Ar[n] * f);
    }
}

template <bool STRUCT>
__device__ __forceinline__ float combine_summary(float f_early, float f_late)
{
    return STRUCT ? f_early * f_late : f_early + f_late;
}

// The whole per-workgroup body for one arithmetic path.
template <bool BF16, bool STRUCT>
__device__ __forceinline__ void scan_segment(
    const ScanKArgs &p, const float *__restrict__ bcp, const float *__restrict__ crp,
    uint32_t *__restrict__ flags,
    float *__restrict__ agg, float *__restrict__ incl, WsHeader *hdr, int64_t seg, int64_t g,
    int w, int lane, float (*s_agg)[kAggFields][kWave], float (*s_part)[kAggFields][kWave],
    float (*s_hin)[kWave], int *s_ctl)
{
    const ScanWsLayout &lay = p.lay;
    const int64_t G = lay.groups;
    const int64_t item = seg * G + g;
    const int64_t b = g / lay.n_dtiles;
    const int64_t dtile = g - b * lay.n_dtiles;
    const int64_t d = dtile * kWave + lane;
    const bool active = d < p.D;
    const int64_t dc = active ? d : (p.D - 1);  // inactive lanes read a valid row
    const int64_t t0 = seg * kSegT + (int64_t)w * kChunkT;
    const int nt = __builtin_amdgcn_readfirstlane((int)max((int64_t)0, min((int64_t)kChunkT, p.L - t0)));
    const bool vec = p.vec && nt == kChunkT;
    const int64_t row_off = (b * p.D + dc) * p.L + t0;
    // prepared B/C rows exist (as zeros) up to the padded length n_seg*kSegT
    const float *bcrow = bcp + (b * lay.n_seg * kSegT + t0) * kBCStride;
    const float *crow = crp + (b * lay.n_seg * kSegT + t0) * kMaxN;
    // Bring this chunk's 32 B/C rows (one 128-byte line each) into L2 with a
    // single vector load (lane l touches half l/32 of row l%32), issued with
    // the x/dt loads.  The per-step scalar loads then hit L2 instead of each
    // paying a full memory latency.
    const float warm = bcrow[(lane & 31) * kBCStride + (lane >> 5) * kMaxN];

    // per-channel constants
    const float bias2 = (p.dt_bias ? p.dt_bias[dc] : 0.f) * kLog2e;
    const float Dd = p.Dskip ? p.Dskip[dc] : 0.f;
    float Ar[kMaxN];
    float a0 = -1.f, inva0 = -1.f;
    if constexpr (STRUCT) {
        a0 = p.A[dc * p.N];
        inva0 = 1.0f / a0;
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            Ar[n] = a0 * (float)(n + 1);
    } else {
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            Ar[n] = (n < p.N) ? p.A[dc * p.N + n] : -1.f;
    }

    // ---- 1. local scan of this wave's chunk from a zero state -------------
    float yl[kChunkT], er[kChunkT];
    float hs[kMaxN];
    float summ;
    {
        float xr[kChunkT], dr[kChunkT];
        load_chunk<BF16>(p.x, row_off, nt, vec, xr, 0.f);
        load_chunk<BF16>(p.dt, row_off, nt, vec, dr, -__builtin_huge_valf());
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            hs[n] = 0.f;
        if constexpr (STRUCT) {
            float E = 1.f;
#pragma unroll
            for (int j = 0; j < kChunkT; ++j) {
                if (j < nt) {  // one basic block per step
                    const float *bc = bcrow + j * kBCStride;  // B, C/(n+1): scalar loads
                    const float l = softplus_log2(fmaf(dr[j], kLog2e, bias2));  // Δ/ln2
                    const float e1 = hw_exp2(a0 * l);                            // exp(Δ A_0)
                    const float xv = xr[j];
                    float en = e1, acc = 0.f;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        if (n)
                            en *= e1;
                        const float pn = bc[n] * xv;
                        const float sn = hs[n] + pn;
                        hs[n] = fmaf(en, sn, -pn);
                        acc = fmaf(bc[kMaxN + n], hs[n], acc);
                    }
                    E *= e1;
                    yl[j] = fmaf(acc, inva0, Dd * xv);
                    er[j] = E;
                }
            }
            summ = E;
            // back to true units: h_n = ĥ_n / A_n
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                hs[n] = hs[n] * (inva0 / (float)(n + 1));
        } else {
            float cumL = 0.f;
#pragma unroll
            for (int j = 0; j < kChunkT; ++j) {
                if (j < nt) {
                    const float *bc = bcrow + j * kBCStride;
                    const float *cr = crow + j * kMaxN;
                    const float l = softplus_log2(fmaf(dr[j], kLog2e, bias2));
                    const float delta = l * kLn2;
                    const float xv = xr[j];
                    cumL += l;
                    float acc = 0.f;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        const float an = Ar[n];
                        const float en = (an == 0.f) ? 1.f : hw_exp2(an * l);
                        const float coef = (an == 0.f) ? delta : expm1f(an * delta) / an;
                        hs[n] = fmaf(en, hs[n], coef * (bc[n] * xv));
                        acc = fmaf(cr[n], hs[n], acc);
                    }
                    yl[j] = fmaf(Dd, xv, acc);
                    er[j] = cumL;
                }
            }
            summ = cumL;
        }
    }

    __asm__ volatile("" ::"v"(warm));  // the warm-up load's value is not needed

    // z is only needed by the final gating: start its loads now so they are in
    // flight while the workgroup resolves its start state
    float zr[kChunkT];
    if (p.z && nt > 0)
        load_chunk<BF16>(p.z, row_off, nt, vec, zr);

    // ---- 2. combine chunk maps inside the workgroup ------------------------
    s_agg[w][0][lane] = summ;
#pragma unroll
    for (int n = 0; n < kMaxN; ++n)
        s_agg[w][1 + n][lane] = hs[n];
    __syncthreads();

    // ---- 3. find which earlier segments' records give this segment's start --
    //  sI     : nearest earlier segment with an inclusive (start-resolved) record,
    //           -1 meaning "the initial state h0"
    //  depth  : number of segments after sI (up to seg-1) whose aggregates
    //           must be folded on top of it
    float F = 0.f, Sg[kMaxN];
    if (w == 0) {
        F = s_agg[0][0][lane];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            Sg[n] = s_agg[0][1 + n][lane];
#pragma unroll
        for (int k = 1; k < kWavesPerSeg; ++k) {
            const float fk = s_agg[k][0][lane];
            float P[kMaxN];
            decay_factors<STRUCT>(fk, Ar, P);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                Sg[n] = fmaf(P[n], Sg[n], s_agg[k][1 + n][lane]);
            F = combine_summary<STRUCT>(F, fk);
        }
        // Fixed association order, independent of scheduling: a segment folds
        // the aggregates of the earlier segments of its superblock, in order,
        // onto the inclusive state that ends the previous superblock.
        const int64_t sI = (seg / kSuperSeg) * kSuperSeg - 1;  // -1 = h0
        const int64_t depth = seg - 1 - sI;
        if (seg + 1 < lay.n_seg) {
            // successors in this superblock fold this segment's aggregate
            float *rec = agg + item * (kAggFields * kWave);
            store_rec(rec + lane, F);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                store_rec(rec + (1 + n) * kWave + lane, Sg[n]);
            publish_flag(flags + item, kFlagAgg, lane);
        }
        if (seg > 0) {
            // wait until the records this segment folds are all published:
            // lane j < depth watches segment seg-1-j (aggregate), lane `depth`
            // watches segment sI (inclusive state; none needed when sI < 0)
            const int64_t s = seg - 1 - lane;
            uint32_t want = 0u;
            if (lane < depth)
                want = kFlagAgg;
            else if (lane == depth && sI >= 0)
                want = kFlagIncl;
            int spins = 0;
            for (;;) {
                const uint32_t f = want ? load_flag(flags + s * G + g) : 0u;
                if (__ballot(f < want) == 0ull)
                    break;
                if (++spins > kSpinLimit) {  // never expected; keeps the kernel finite
                    if (lane == 0)
                        atomicOr(&hdr->error, kErrSpinTimeout);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) {
            s_ctl[0] = sI;
            s_ctl[1] = depth;
        }
    }
    __syncthreads();

    // ---- 4. fold the predecessors' aggregates, four waves in parallel --------
    const int64_t sI = __builtin_amdgcn_readfirstlane((int)s_ctl[0]);
    const int64_t depth = __builtin_amdgcn_readfirstlane((int)s_ctl[1]);
    {
        const int64_t per = (depth + kWavesPerSeg - 1) / kWavesPerSeg;
        const int64_t lo = min(depth, (int64_t)w * per), hi = min(depth, lo + per);
        float pf = STRUCT ? 1.f : 0.f;  // identity map
        float ps[kMaxN];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            ps[n] = 0.f;
        for (int64_t j = lo; j < hi; j += 2) {
            // two records per round trip; records are in time order
            const bool two = j + 1 < hi;
            const float *r0 = agg + ((sI + 1 + j) * G + g) * (kAggFields * kWave);
            const float *r1 = two ? r0 + G * (kAggFields * kWave) : r0;
            float f0 = load_rec(r0 + lane), f1 = load_rec(r1 + lane);
            float v0[kMaxN], v1[kMaxN];
#pragma unroll
            for (int n = 0; n < kMaxN; ++n) {
                v0[n] = load_rec(r0 + (1 + n) * kWave + lane);
                v1[n] = load_rec(r1 + (1 + n) * kWave + lane);
            }
            float P[kMaxN];
            decay_factors<STRUCT>(f0, Ar, P);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                ps[n] = fmaf(P[n], ps[n], v0[n]);
            pf = combine_summary<STRUCT>(pf, f0);
            if (two) {
                decay_factors<STRUCT>(f1, Ar, P);
#pragma unroll
                for (int n = 0; n < kMaxN; ++n)
                    ps[n] = fmaf(P[n], ps[n], v1[n]);
                pf = combine_summary<STRUCT>(pf, f1);
            }
        }
        s_part[w][0][lane] = pf;
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            s_part[w][1 + n][lane] = ps[n];
    }
    __syncthreads();

    // ---- 5. segment start state, inclusive record, per-wave start state -----
    if (w == 0) {
        float hin[kMaxN];
        if (sI < 0) {
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                hin[n] = (p.h0 && n < p.N) ? p.h0[(b * p.D + dc) * p.N + n] : 0.f;
        } else {
            const float *rec = incl + (sI * G + g) * (kInclFields * kWave);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                hin[n] = load_rec(rec + n * kWave + lane);
        }
#pragma unroll
        for (int k = 0; k < kWavesPerSeg; ++k) {
            float P[kMaxN];
            decay_factors<STRUCT>(s_part[k][0][lane], Ar, P);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                hin[n] = fmaf(P[n], hin[n], s_part[k][1 + n][lane]);
        }
        float P[kMaxN];
        decay_factors<STRUCT>(F, Ar, P);
        float hout[kMaxN];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            hout[n] = fmaf(P[n], hin[n], Sg[n]);
        if (seg + 1 < lay.n_seg && (seg + 1) % kSuperSeg == 0) {
            float *rec = incl + item * (kInclFields * kWave);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                store_rec(rec + n * kWave + lane, hout[n]);
            publish_flag(flags + item, kFlagIncl, lane);
        }
        if (seg + 1 == lay.n_seg && p.h_last && active) {
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                if (n < p.N)
                    p.h_last[(b * p.D + d) * p.N + n] = hout[n];
        }
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            s_hin[n][lane] = hin[n];
    }
    __syncthreads();

    if (nt <= 0)
        return;

    // ---- 6. this wave's start state, fix-up, gate, store -------------------
    float hin[kMaxN];
#pragma unroll
    for (int n = 0; n < kMaxN; ++n)
        hin[n] = s_hin[n][lane];
    for (int k = 0; k < w; ++k) {
        float P[kMaxN];
        decay_factors<STRUCT>(s_agg[k][0][lane], Ar, P);
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            hin[n] = fmaf(P[n], hin[n], s_agg[k][1 + n][lane]);
    }
    const bool zero_start = (seg == 0 && w == 0 && p.h0 == nullptr);
    // The step conditions of the fix-up loops must not be shared with the scan
    // loops (keeping 32 condition masks alive costs scalar registers): give the
    // compiler a copy of nt it cannot prove equal.
    int ntf = nt;
    __asm__ volatile("" : "+s"(ntf));

    if constexpr (STRUCT) {
        // coefficient of the carried state in scaled units: (n+1) A_0 h_in,n
        float hsc[kMaxN];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            hsc[n] = Ar[n] * hin[n];
        if (!zero_start) {
#pragma unroll
            for (int j = 0; j < kChunkT; ++j) {
                if (j < ntf) {
                    const float *cs = bcrow + j * kBCStride + kMaxN;  // C/(n+1)
                    const float Ej = er[j];
                    float qh = 0.f;
#pragma unroll
                    for (int n = kMaxN - 1; n >= 0; --n)
                        qh = fmaf(qh, Ej, cs[n] * hsc[n]);
                    yl[j] = fmaf(qh * Ej, inva0, yl[j]);
                }
            }
        }
        if (p.z) {
#pragma unroll
            for (int j = 0; j < kChunkT; ++j)
                yl[j] *= silu_hw(zr[j]);
        }
    } else {
        if (!zero_start) {
#pragma unroll
            for (int j = 0; j < kChunkT; ++j) {
                if (j < ntf) {
                    const float *cr = crow + j * kMaxN;
                    const float Lj = er[j];
                    float corr = 0.f;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        const float gdec = (Ar[n] == 0.f) ? 1.f : hw_exp2(Ar[n] * Lj);
                        corr = fmaf(cr[n] * gdec, hin[n], corr);
                    }
                    yl[j] += corr;
                }
            }
        }
        if (p.z) {
#pragma unroll
            for (int j = 0; j < kChunkT; ++j)
                yl[j] *= silu_hw(zr[j]);
        }
    }
    if (active)
        store_chunk<BF16>(p.y, row_off, nt, vec, yl);
}

template <bool BF16>
__global__ void __launch_bounds__(kWave *kWavesPerSeg, 3) scan_main_kernel(
    ScanKArgs p, const float *__restrict__ bcp, const float *__restrict__ crp,
    const uint32_t *__restrict__ tiles)
{
    __shared__ float s_agg[kWavesPerSeg][kAggFields][kWave];
    __shared__ float s_part[kWavesPerSeg][kAggFields][kWave];
    __shared__ float s_hin[kMaxN][kWave];
    __shared__ int s_ctl[2];
    __shared__ uint32_t s_ticket;

    WsHeader *hdr = reinterpret_cast<WsHeader *>(p.ws + p.lay.off_header);
    uint32_t *flags = reinterpret_cast<uint32_t *>(p.ws + p.lay.off_flags);
    float *agg = reinterpret_cast<float *>(p.ws + p.lay.off_agg);
    float *incl = reinterpret_cast<float *>(p.ws + p.lay.off_incl);

    if (threadIdx.x == 0)
        s_ticket = atomicAdd(&hdr->ticket, 1u);
    __syncthreads();
    const int64_t item = (int64_t)__builtin_amdgcn_readfirstlane(s_ticket);
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int64_t seg = item / p.lay.groups;
    const int64_t g = item - seg * p.lay.groups;
    const int64_t dtile = g % p.lay.n_dtiles;
    const uint32_t path = __builtin_amdgcn_readfirstlane(tiles[dtile]);
    if (path == kPathStructured)
        scan_segment<BF16, true>(p, bcp, crp, flags, agg, incl, hdr, seg, g, w, lane, s_agg, s_part,
                                 s_hin, s_ctl);
    else
        scan_segment<BF16, false>(p, bcp, crp, flags, agg, incl, hdr, seg, g, w, lane, s_agg,
                                  s_part, s_hin, s_ctl);
}

// Writes h_last = h0 (or zeros) for an empty sequence (L == 0).
__global__ void copy_or_zero_kernel(const float *__restrict__ src, float *__restrict__ dst,
                                    int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        dst[i] = src ? src[i] : 0.f;
}

}  // namespace

ScanWsLayout scan_ws_layout(int64_t B, int64_t D, int64_t L)
{
    ScanWsLayout l;
    l.n_dtiles = (D + kWave - 1) / kWave;
    l.groups = B * l.n_dtiles;
    l.n_seg = (L + kSegT - 1) / kSegT;
    l.n_items = l.groups * l.n_seg;
    size_t off = 0;
    l.off_header = off;
    off += 256;
    l.off_flags = off;
    off = round_up(off + (size_t)l.n_items * 4, 256);
    l.off_tiles = off;
    off = round_up(off + (size_t)l.n_dtiles * 4, 256);
    l.off_bc = off;
    off = round_up(off + (size_t)B * (size_t)(l.n_seg * kSegT) * kBCStride * 4, 256);
    l.off_craw = off;
    off = round_up(off + (size_t)B * (size_t)(l.n_seg * kSegT) * kMaxN * 4, 256);
    l.off_agg = off;
    off = round_up(off + (size_t)l.n_items * kAggFields * kWave * 4, 256);
    l.off_incl = off;
    off = round_up(off + (size_t)l.n_items * kInclFields * kWave * 4, 256);
    l.total = off;
    return l;
}

hipError_t launch_selective_scan(const ScanArgs &a, hipStream_t s)
{
    const ScanWsLayout &lay = a.lay;
    if (a.L == 0) {
        if (a.h_last) {
            const int64_t n = a.B * a.D * a.N;
            hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)),
                               dim3(256), 0, s, a.h0, a.h_last, n);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    if (lay.n_items == 0)
        return hipSuccess;
    // prep
    const int64_t n_zero = lay.n_items > 0 ? lay.n_items : 1;
    const int64_t n_bc = a.B * lay.n_seg * kSegT * kMaxN;
    const int64_t classify_base = (n_zero + n_bc + kWave - 1) / kWave * kWave;
    const int64_t total = classify_base + lay.n_dtiles * kWave;
    const unsigned prep_blocks = (unsigned)((total + 255) / 256);
    if (a.bf16)
        hipLaunchKernelGGL(scan_prep_kernel<true>, dim3(prep_blocks), dim3(256), 0, s, a.Bm,
                           a.Cm, a.A, a.ws, lay, a.D, a.L, a.N, n_zero, n_bc, classify_base);
    else
        hipLaunchKernelGGL(scan_prep_kernel<false>, dim3(prep_blocks), dim3(256), 0, s, a.Bm,
                           a.Cm, a.A, a.ws, lay, a.D, a.L, a.N, n_zero, n_bc, classify_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;

    ScanKArgs k;
    k.x = a.x;
    k.dt = a.dt;
    k.z = a.z;
    k.y = a.y;
    k.dt_bias = a.dt_bias;
    k.A = a.A;
    k.Dskip = a.Dskip;
    k.h0 = a.h0;
    k.h_last = a.h_last;
    k.ws = a.ws;
    k.lay = lay;
    k.B = a.B;
    k.D = a.D;
    k.L = a.L;
    k.N = a.N;
    const size_t esz = a.bf16 ? 2 : 4;
    const uintptr_t amask = (uintptr_t)a.x | (uintptr_t)a.dt | (uintptr_t)a.y |
                            (uintptr_t)(a.z ? a.z : a.x);
    k.vec = ((amask & 15u) == 0 && ((size_t)a.L * esz) % 16 == 0) ? 1 : 0;
    const float *bcp = reinterpret_cast<const float *>(a.ws + lay.off_bc);
    const float *crp = reinterpret_cast<const float *>(a.ws + lay.off_craw);
    const uint32_t *tiles = reinterpret_cast<const uint32_t *>(a.ws + lay.off_tiles);
    if (a.ev_start)
        hipEventRecord(a.ev_start, s);
    if (a.bf16)
        hipLaunchKernelGGL(scan_main_kernel<true>, dim3((unsigned)lay.n_items),
                           dim3(kWave * kWavesPerSeg), 0, s, k, bcp, crp, tiles);
    else
        hipLaunchKernelGGL(scan_main_kernel<false>, dim3((unsigned)lay.n_items),
                           dim3(kWave * kWavesPerSeg), 0, s, k, bcp, crp, tiles);
    e = hipGetLastError();
    if (a.ev_stop)
        hipEventRecord(a.ev_stop, s);
    return e;
}

}  // namespace mamba
