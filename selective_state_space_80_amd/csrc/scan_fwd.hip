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
//     are the same for all 64 lanes: the 128 steps of a segment are staged in
//     LDS once per workgroup and read back with broadcast LDS loads.
//   * Work is cut into segments of kSegT = 4 x 32 steps.  Each of the 4 waves of
//     a workgroup scans one 32-step chunk from a zero state, keeping its 32
//     partial outputs and decay factors in registers (fully unrolled loop).
//   * The end state of a chunk is an affine map h -> P h + S of its start state
//     (the block-wise scan with a prefix state handed to later blocks,
//     "Mamba: Linear-Time Sequence Modeling with Selective SSMs", selective scan
//     section).  Chunk maps are combined in LDS inside the workgroup.  Across
//     workgroups every segment publishes its map (an aggregate record) in the
//     workspace; segments are grouped 8 to a superblock, and the last segment
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
//   * Every global load a wave needs before its scan is issued before the
//     first of them is waited for: the small ones (conv taps, B/C rows) first,
//     then the chunk's x and dt, so that waiting for the small ones (the wait
//     counter is in order) leaves the chunk's loads in flight.  A branch
//     around a load works against this: at the join the compiler may reuse a
//     register an in-flight load still targets and so wait for every load.
//     fp32 problems of whole segments with aligned rows therefore take a FULL
//     instantiation with no ragged-chunk path at all.
//
// Two arithmetic paths, chosen per 64-channel tile by the prep kernel:
//   structured  A_dn = (n+1) A_d0 exactly with A_d0 <= -1 (the S4D-real form;
//               smaller |A_d0| loses accuracy in e - 1, see kStructMaxA0).
//               Then exp(Δ A_dn) = e^(n+1) with e = exp(Δ A_d0): one exp per
//               element, powers by multiplication.  The state is kept scaled,
//               ĥ_n = A_dn h_n, which turns the ZOH update into
//               ĥ <- ĥ + (e_n - 1)(ĥ + B_n x)   (exact algebra of
//               h <- e_n h + (e_n - 1)/A_n B_n x), so no division per state; the
//               readout uses C_n/(n+1) (scaled while B, C are staged) and 1/A_d0
//               per channel.  4 VALU operations per state and step.
//   general     any A: per state exp and the ZOH input coefficient
//               (exp(ΔA_n) - 1)/A_n, by series near ΔA_n = 0 (which includes the
//               A_n = 0 limit Δ).  Slower, exact form.
#include <cstddef>

#include "device_common.h"
#include "internal.h"

namespace mamba {

namespace {

struct WsHeader {
    uint32_t ticket;
    uint32_t error;  // bit 0: a carry wait timed out (read by mamba_selective_scan_check)
    uint32_t epoch;  // call counter (never 0): tag of this call's inclusive records
    uint32_t pad[61];
};
static_assert(offsetof(WsHeader, error) == kScanErrorWordOffset, "error word of the header");

constexpr uint32_t kFlagAgg = 1u;
constexpr uint32_t kErrSpinTimeout = 1u;
// Segments per superblock of the carry when a problem has few 64-channel
// groups (16 or 32 measured 1-8% slower on the three forward workloads, 4 or 6
// within 1%).  With at least kChainGroups groups, consecutive segments of a
// group are about one round of resident workgroups apart, so each segment
// reads only its predecessor's end state (a chain, superblocks of one).
constexpr int64_t kSuperSeg = 8;
// The structured update forms e - 1 = 2^w - 1 (w = ΔA_0 log2 e) by subtraction,
// so the exponential's rounding becomes an error of about one ulp / |w| in each
// step's increment, and it accumulates along the sequence.  With A_0 = -1 (the
// S4D-real form) that stays far inside the fp32 tolerance; at A_0 = -1/16 an
// fp32 scan of 4096 steps already missed it (4.6e-4).  Tiles with a smaller
// |A_0| take the general path, whose input coefficient comes from a series near
// 0 and whose state is not scaled by A.
constexpr float kStructMaxA0 = -1.0f;
constexpr int64_t kChainGroups = 384;
// waves per SIMD the register budget is held to (158-167 VGPRs)
constexpr int kScanWavesPerSimd = 3;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Prep kernel: clears the ticket, the error word and the per-segment flags,
// zeroes the tags of every inclusive record the main kernel will poll, and
// decides per 64-channel tile whether A has the structured form (with
// A_0 <= kStructMaxA0).
__global__ void __launch_bounds__(256) scan_prep_kernel(const float *__restrict__ A,
                                                        unsigned char *__restrict__ ws,
                                                        ScanWsLayout lay, int64_t D, int N,
                                                        int64_t n_flags, int64_t classify_base,
                                                        int64_t clear_base, int64_t n_clear16,
                                                        int keep_error)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= clear_base) {
        // Polled inclusive records start this call with tag 0, which no call
        // uses, so a word carries this call's epoch only once this call has
        // written it, whatever the workspace's memory held before.
        const int64_t k = i - clear_base;
        if (k < n_clear16)
            reinterpret_cast<uint4 *>(ws + lay.off_incl)[k] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    if (i < n_flags) {
        if (i == 0) {
            WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + lay.off_header);
            hdr->ticket = 0u;
            if (!keep_error)
                hdr->error = 0u;
            const uint32_t e = hdr->epoch + 1u;
            hdr->epoch = e ? e : 1u;
        }
        reinterpret_cast<uint32_t *>(ws + lay.off_flags)[i] = 0u;
        return;
    }
    const int64_t c = i - classify_base;  // classify region starts on a wave boundary
    if (c < 0 || c >= lay.n_dtiles * kWave)
        return;
    const int64_t d = c;
    bool ok = true;
    if (d < D) {
        // all loads first (no short-circuit), then the comparisons
        float a[kMaxN];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            a[n] = (n < N) ? A[d * N + n] : 0.f;
        ok = (a[0] <= kStructMaxA0) && (a[0] > -1e30f);
#pragma unroll
        for (int n = 1; n < kMaxN; ++n)
            ok = ok & ((n >= N) | (a[n] == (float)(n + 1) * a[0]));
    }
    const uint64_t bad = __ballot(!ok);
    if ((threadIdx.x & (kWave - 1)) == 0)
        reinterpret_cast<uint32_t *>(ws + lay.off_tiles)[c / kWave] =
            bad ? kPathGeneral : kPathStructured;
}

// ---------------------------------------------------------------------------
// Per-lane chunk inputs: 32 consecutive time steps of one row.  `vec` means the
// chunk is full and the row is 16-byte aligned, so 128-bit loads are used.
// Steps at or past L are filled with `pad` and never stored: padding x with 0
// and dt with -inf makes such a step an exact identity of the recurrence
// (step 0, decay 1, no input).
// Register budget: bf16 inputs stay packed two steps per register (16 VGPRs
// for the chunk); fp32 inputs take 32 VGPRs, but a step's input register dies
// at the step that writes the step's output, so inputs and outputs share
// registers.  Each lane's chunk is one whole 128-byte line (fp32) or half of
// one whose other half the neighbouring wave loads at the same time (bf16):
// every line is fetched from memory once.
template <bool BF16> struct InChunk;

template <> struct InChunk<true> {
    uint32_t w[kChunkT / 2];  // step 2i in the low half, 2i+1 in the high half
    // slots [klo, khi) come from base + off + slot, the others are `pad`
    __device__ __forceinline__ void load(const void *base, int64_t off, int klo, int khi, bool vec,
                                         float pad)
    {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + off;
        if (vec) {
            const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 8; ++i) {
                const uint4 a = q[i];
                w[4 * i + 0] = a.x;
                w[4 * i + 1] = a.y;
                w[4 * i + 2] = a.z;
                w[4 * i + 3] = a.w;
            }
        } else {
            const uint32_t pb = __float_as_uint(pad) >> 16;
#pragma unroll
            for (int i = 0; i < kChunkT / 2; ++i) {
                const uint32_t lo = (2 * i >= klo && 2 * i < khi) ? (uint32_t)p[2 * i] : pb;
                const uint32_t hi =
                    (2 * i + 1 >= klo && 2 * i + 1 < khi) ? (uint32_t)p[2 * i + 1] : pb;
                w[i] = lo | (hi << 16);
            }
        }
    }
    __device__ __forceinline__ float get(int j) const
    {
        return (j & 1) ? __uint_as_float(w[j >> 1] & 0xffff0000u)
                       : __uint_as_float(w[j >> 1] << 16);
    }
};

template <> struct InChunk<false> {
    float v[kChunkT];
    // slots [klo, khi) come from base + off + slot, the others are `pad`
    __device__ __forceinline__ void load(const void *base, int64_t off, int klo, int khi, bool vec,
                                         float pad)
    {
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
                v[i] = (i >= klo && i < khi) ? p[i] : pad;
        }
    }
    __device__ __forceinline__ float get(int j) const { return v[j]; }
};

// Stores slots [klo, khi) of a chunk, slot k's value being val(k), to
// base + off + k; with `accumulate` each value is added to what is there.
template <bool BF16, typename Val>
__device__ __forceinline__ void store_chunk(void *base, int64_t off, int klo, int khi, bool vec,
                                            bool accumulate, Val val)
{
    if constexpr (!BF16) {
        float *p = reinterpret_cast<float *>(base) + off;
        if (vec) {
            float4 *q = reinterpret_cast<float4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 4; ++i) {
                float4 o = make_float4(val(4 * i), val(4 * i + 1), val(4 * i + 2), val(4 * i + 3));
                if (accumulate) {
                    const float4 old = q[i];
                    o = make_float4(o.x + old.x, o.y + old.y, o.z + old.z, o.w + old.w);
                }
                q[i] = o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kChunkT; ++i)
                if (i >= klo && i < khi)
                    p[i] = accumulate ? p[i] + val(i) : val(i);
        }
    } else {
        uint16_t *p = reinterpret_cast<uint16_t *>(base) + off;
        if (vec) {
            uint4 *q = reinterpret_cast<uint4 *>(p);
#pragma unroll
            for (int i = 0; i < kChunkT / 8; ++i) {
                uint32_t old4[4] = {0u, 0u, 0u, 0u};
                if (accumulate) {
                    const uint4 o = q[i];
                    old4[0] = o.x;
                    old4[1] = o.y;
                    old4[2] = o.z;
                    old4[3] = o.w;
                }
                uint32_t w4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float lo = val(8 * i + 2 * k), hi = val(8 * i + 2 * k + 1);
                    if (accumulate) {
                        lo += __uint_as_float(old4[k] << 16);
                        hi += __uint_as_float(old4[k] & 0xffff0000u);
                    }
                    w4[k] = cvt2(lo, hi);
                }
                q[i] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kChunkT; ++i)
                if (i >= klo && i < khi) {
                    const float o = accumulate ? bf16_bits_to_f32(p[i]) + val(i) : val(i);
                    p[i] = (uint16_t)f32_to_bf16_bits(o);
                }
        }
    }
}

// Carry records between workgroups.  Every record word and every flag is
// accessed with agent-scope relaxed atomics, which are coherent across the
// XCDs' L2 caches without whole-cache write-back or invalidation.  A writer of
// a segment aggregate waits until all of its record stores have completed
// (vmcnt = 0) before it stores the flag; a reader loads record words only
// after it has seen the flag, so it reads this call's values.
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

// Inclusive records (the superblock-to-superblock chain, on the critical path
// of long sequences) instead carry the call's epoch in the high half of every
// 64-bit word, beside the value: a reader accepts a word once its tag is this
// call's, so the record needs no flag, its writer no wait for its stores, and
// its reader one round trip.  Each 64-bit word is written and read
// atomically.  The prep kernel of the same call has set the tag of every
// polled word to 0 and the epoch is never 0, so only a word this call wrote
// can match, whatever the workspace's memory held before the call.
__device__ __forceinline__ void store_tagged(uint64_t *p, float v, uint32_t epoch)
{
    const uint64_t w = ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_tagged(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish_flag(uint32_t *p, uint32_t v, int lane)
{
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin (with sleeps) until the flag at `p` reaches `want` in every lane that
// wants one (want = 0: nothing to wait for).  Bounded by `limit` polls: a
// timeout is recorded in the workspace header, the caller poisons what it
// computes from the unfinished data (NaN), and the kernel carries on, so it
// always ends.  Returns false on a timeout.
__device__ __forceinline__ bool wait_flags(const uint32_t *p, uint32_t want, WsHeader *hdr,
                                           int lane, int limit)
{
    int spins = 0;
    for (;;) {
        const uint32_t f = want ? load_flag(p) : 0u;
        if (__ballot(f < want) == 0ull)
            return true;
        if (++spins > limit) {  // not expected with the default limit
            if (lane == 0)
                atomicOr(&hdr->error, kErrSpinTimeout);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

struct ScanKArgs {
    const void *x, *dt, *z, *Bm, *Cm;
    void *y;
    const float *dt_bias, *A, *Dskip, *h0;
    float *h_last;
    unsigned char *ws;
    ScanWsLayout lay;
    int64_t B, D, L;
    int N;
    int vec;     // rows of x, dt, z, y are 16-byte aligned for vector access
    int bc_vec;  // N == 16 and B, C 16-byte aligned: rows staged with 128-bit loads
    // fused front end (CONV instantiation only): x holds the raw input
    const float *conv_w, *conv_b;
    const void *conv_state_in;  // [B, D, K-1] raw inputs before t = 0, or NULL (zeros)
    int conv_K;
    int accumulate;       // y += result instead of y = result
    float *chunk_states;  // per 32-step chunk its start state, or NULL (see launch)
    int64_t n_cslots;     // chunk slots per group in chunk_states
    int spin_limit;       // polls before a carry wait gives up
};

// The fused front end's per-lane inputs besides the chunk itself: the taps,
// the bias and the raw inputs of the three steps before the chunk (from x, or
// from the carried conv state before t = 0).
template <bool BF16>
struct ConvPre {
    float wk[kFusedConvTaps], cb;
    float vx[kFusedConvTaps - 1], vs[kFusedConvTaps - 1];
    bool in_x[kFusedConvTaps - 1], in_cs[kFusedConvTaps - 1];
    // every load from an index that is always valid, with no branch around
    // any of them; the values are selected where they are used
    __device__ __forceinline__ void load(const ScanKArgs &p, int64_t bd, int64_t dc, int64_t t0,
                                         int64_t row_off)
    {
        using E = Elem<BF16>;
        using T = typename E::T;
        const int K = p.conv_K;
#pragma unroll
        for (int s = 0; s < kFusedConvTaps; ++s) {
            const int k = s - (kFusedConvTaps - K);
            wk[s] = p.conv_w[dc * K + (k >= 0 ? k : 0)];
        }
        cb = (p.conv_b ? p.conv_b : p.conv_w)[dc];  // conv_w has >= D entries
        const T *xs = reinterpret_cast<const T *>(p.x);
        const T *cs = reinterpret_cast<const T *>(p.conv_state_in ? p.conv_state_in : p.x);
#pragma unroll
        for (int i = 0; i < kFusedConvTaps - 1; ++i) {
            const int64_t t = t0 - (kFusedConvTaps - 1) + i;
            const int64_t si = (int64_t)(K - 1) + t;  // slot of the carried raw inputs (t < 0)
            in_x[i] = t >= 0 && t < p.L;
            in_cs[i] = t < 0 && p.conv_state_in && si >= 0;
            vx[i] = E::load(xs + (in_x[i] ? row_off - (kFusedConvTaps - 1) + i : 0));
            vs[i] = E::load(cs + (in_cs[i] ? bd * (K - 1) + si : 0));
        }
    }
};

// Fused front end: the chunk's scan inputs SiLU(bias + sum_k w_k x_(t-K+1+k))
// from the raw inputs of the chunk (in `xin`) and of the three steps before it
// (in `cp`).  Taps are right-aligned in kFusedConvTaps slots (zero weights in
// front for K < 4).  Computed from the last step down, so each raw value is
// still available when the outputs that need it are formed.  Steps at or past
// the end of the sequence get the identity input 0.
template <bool BF16>
__device__ __forceinline__ void conv_chunk(const ScanKArgs &p, const ConvPre<BF16> &cp,
                                           const InChunk<BF16> &xin, int nt, float (&xc)[kChunkT])
{
    const int K = p.conv_K;
    float wk[kFusedConvTaps], hm[kFusedConvTaps - 1];
#pragma unroll
    for (int s = 0; s < kFusedConvTaps; ++s)
        wk[s] = s - (kFusedConvTaps - K) >= 0 ? cp.wk[s] : 0.f;
    const float cb = p.conv_b ? cp.cb : 0.f;
#pragma unroll
    for (int i = 0; i < kFusedConvTaps - 1; ++i)
        hm[i] = cp.in_x[i] ? cp.vx[i] : (cp.in_cs[i] ? cp.vs[i] : 0.f);
    auto raw = [&](int i) -> float { return i >= 0 ? xin.get(i) : hm[kFusedConvTaps - 1 + i]; };
#pragma unroll
    for (int j = kChunkT - 1; j >= 0; --j) {
        float acc = cb;
#pragma unroll
        for (int s = 0; s < kFusedConvTaps; ++s)
            acc = fmaf(wk[s], raw(j - (kFusedConvTaps - 1) + s), acc);
        xc[j] = (j < nt) ? silu_hw(acc) : 0.f;
    }
}

// The segment's B_t (s_bc[0]) and C_t (s_bc[1]; C_t,n/(n+1) on the structured
// path) for its kSegT steps, as fp32 rows of kMaxN: zero past N and past L.
// Whole segments with N = 16 and aligned rows take two 128-bit loads per
// thread and matrix (fp32) or one (bf16).
template <bool BF16, bool STRUCT, bool REV, bool ADJ>
__device__ __forceinline__ void stage_bc(const ScanKArgs &p, float (*s_bc)[kSegT][kMaxN],
                                         int64_t b, int64_t seg, int64_t Ls, int tid)
{
    using E = Elem<BF16>;
    using T = typename E::T;
    constexpr int kThreads = kWave * kWavesPerSeg;
    const int64_t t0s = seg * kSegT;  // first step of the segment (in scan order)
    // Step s of the scan order is memory row s forward and row Ls-1-s in
    // reverse (Ls = L rounded up to whole chunks; rows >= L are padding, zero).
    // A whole segment is one run of kSegT rows; in reverse the run ends at the
    // segment's first step and its rows come in the opposite order.
    const int64_t run0 = REV ? Ls - t0s - kSegT : t0s;
    const bool whole = REV ? (run0 >= 0 && Ls - t0s <= p.L) : (t0s + kSegT <= p.L);
    auto lrow = [](int pr) { return REV ? kSegT - 1 - pr : pr; };  // run row -> LDS row
    // the adjoint scan's input rows are C (in the first LDS matrix)
    const T *Bb = reinterpret_cast<const T *>(ADJ ? p.Cm : p.Bm) + b * p.L * p.N;
    const T *Cb = reinterpret_cast<const T *>(p.Cm) + b * p.L * p.N;
    auto cscale = [](float c, int n) -> float {
        return STRUCT ? c * hw_rcp((float)(n + 1)) : c;
    };
    if (p.bc_vec && whole) {
        const T *src[2] = {Bb + run0 * p.N, Cb + run0 * p.N};
        if constexpr (!BF16) {
            constexpr int kPer = kSegT * kMaxN / 4 / kThreads;  // float4 per thread and matrix
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const int q = tid + i * kThreads;
                    const int row = lrow(q >> 2), n4 = (q & 3) * 4;
                    float4 v = reinterpret_cast<const float4 *>(src[m])[q];
                    if (m == 1)
                        v = make_float4(cscale(v.x, n4), cscale(v.y, n4 + 1),
                                        cscale(v.z, n4 + 2), cscale(v.w, n4 + 3));
                    *reinterpret_cast<float4 *>(&s_bc[m][row][n4]) = v;
                }
            }
        } else {
            static_assert(kSegT * kMaxN / 8 == kThreads, "one 8-value load per thread");
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int row = lrow(tid >> 1), n8 = (tid & 1) * 8;
                const uint4 a = reinterpret_cast<const uint4 *>(src[m])[tid];
                const uint32_t w4[4] = {a.x, a.y, a.z, a.w};
                float v[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[2 * k] = __uint_as_float(w4[k] << 16);
                    v[2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
                }
                if (m == 1) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        v[k] = cscale(v[k], n8 + k);
                }
                float4 *dst = reinterpret_cast<float4 *>(&s_bc[m][row][n8]);
                dst[0] = make_float4(v[0], v[1], v[2], v[3]);
                dst[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
    } else {
        for (int e = tid; e < 2 * kSegT * kMaxN; e += kThreads) {
            const int m = e / (kSegT * kMaxN);
            const int r = (e / kMaxN) % kSegT, n = e % kMaxN;
            float v = 0.f;
            const int64_t t = REV ? Ls - 1 - (t0s + r) : t0s + r;
            if (n < p.N && t >= 0 && t < p.L)
                v = E::load((m ? Cb : Bb) + t * p.N + n);
            s_bc[m][r][n] = m ? cscale(v, n) : v;
        }
    }
}

// B/C of a whole segment with N = 16 and aligned rows, fp32: loaded into
// registers first, stored to LDS once the chunk's own loads are issued.
template <bool STRUCT, bool REV, bool ADJ>
struct BcPre {
    static constexpr int kPer = kSegT * kMaxN / 4 / (kWave * kWavesPerSeg);
    float4 v[2][kPer];
    __device__ __forceinline__ void load(const ScanKArgs &p, int64_t b, int64_t seg, int64_t Ls,
                                         int tid)
    {
        const int64_t t0s = seg * kSegT;
        const int64_t run0 = REV ? Ls - t0s - kSegT : t0s;
        const float *Bb = reinterpret_cast<const float *>(ADJ ? p.Cm : p.Bm) + b * p.L * p.N;
        const float *Cb = reinterpret_cast<const float *>(p.Cm) + b * p.L * p.N;
        const float *src[2] = {Bb + run0 * p.N, Cb + run0 * p.N};
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                v[m][i] = reinterpret_cast<const float4 *>(src[m])[tid + i * (kWave * kWavesPerSeg)];
    }
    __device__ __forceinline__ void store(float (*s_bc)[kSegT][kMaxN], int tid) const
    {
        auto lrow = [](int pr) { return REV ? kSegT - 1 - pr : pr; };
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int q = tid + i * (kWave * kWavesPerSeg);
                const int row = lrow(q >> 2), n4 = (q & 3) * 4;
                float4 x = v[m][i];
                if (m == 1 && STRUCT)
                    x = make_float4(x.x * hw_rcp((float)(n4 + 1)), x.y * hw_rcp((float)(n4 + 2)),
                                    x.z * hw_rcp((float)(n4 + 3)), x.w * hw_rcp((float)(n4 + 4)));
                *reinterpret_cast<float4 *>(&s_bc[m][row][n4]) = x;
            }
        }
    }
};

// One LDS row of kMaxN floats into registers (four 128-bit broadcast reads).
__device__ __forceinline__ void lds_row(const float *row, float (&v)[kMaxN])
{
#pragma unroll
    for (int q = 0; q < kMaxN / 4; ++q) {
        const float4 t = reinterpret_cast<const float4 *>(row)[q];
        v[4 * q + 0] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
    }
}

// Apply the chunk map (f, S) to a state: h_n <- P_n(f) h_n + S_n, where
//   structured: f = prod of e over the chunk, P_n = f^(n+1)
//   general:    f = sum over the chunk of Δ/ln2, P_n = 2^(A_n f)   (A_n = 0 -> 1)
// S_n is read through `get(n)` so it can come from registers, LDS or a record.
// e = 2^w and e - 1 for a structured step's decay exponent w = Δ A_0 / ln2.
// Near w = 0 the exponential carries about an ulp of 1, which in e - 1 formed
// by subtraction is a relative error of ~6e-8 / |w ln2|; every state's
// increment (e_n - 1)(ĥ + B x) inherits it, and along a sequence of small steps
// it accumulates in the state.  So for |w ln2| < 1/64, e - 1 is the series
// u + u^2/2 + u^3/6 (u = w ln2; truncation below 2e-7 relative) and e = 1 + that,
// rounded once; beyond, e is the exponential and e - 1 its subtraction.
__device__ __forceinline__ void step_decay(float w, float &e, float &em1)
{
    constexpr float c1 = 0.693147180559945309f;  // ln 2
    constexpr float c2 = c1 * c1 / 2.f, c3 = c1 * c1 * c1 / 6.f;
    const float x = hw_exp2(w);
    const float sr = w * fmaf(fmaf(c3, w, c2), w, c1);
    const bool small = fabsf(w) < (1.f / 64.f) * 1.44269504088896341f;
    em1 = small ? sr : x - 1.f;
    e = small ? 1.f + sr : x;
}

// One channel's row of A held in LDS ([n][lane] layout): Ar[n].
struct ARow {
    const float (*a)[kWave];
    int lane;
    __device__ __forceinline__ float operator[](int n) const { return a[n][lane]; }
};

// Applies a span's map h <- P h + S to h.  The span's decay is carried as the
// sum f of its steps' exponents: Σ Δ A_0 / ln2 on the structured path, whose
// state n decays by P_n = 2^((n+1) f), and Σ Δ / ln2 on the general path,
// P_n = 2^(A_n f).  One exponential per state keeps each P_n within about an ulp
// however many steps the span holds; powers of the span's decay, formed by
// products, would carry n+1 times its rounding into every later segment.
template <bool STRUCT, typename GetS>
__device__ __forceinline__ void apply_map(float f, GetS get, const ARow &Ar, float (&h)[kMaxN])
{
    const float fc = fminf(f, __FLT_MAX__);  // finite: A_n = 0 gives 2^0 = 1
#pragma unroll
    for (int n = 0; n < kMaxN; ++n) {
        const float P = STRUCT ? hw_exp2(f * (float)(n + 1)) : hw_exp2(Ar[n] * fc);
        h[n] = fmaf(P, h[n], get(n));
    }
}

// The decay summary of two consecutive spans: exponent sums add.
__device__ __forceinline__ float combine_summary(float f_early, float f_late)
{
    return f_early + f_late;
}

// The whole per-workgroup body for one arithmetic path.
template <bool BF16, bool STRUCT, bool CONV, bool REV, bool ADJ, bool FULL>
__device__ __forceinline__ void scan_segment(
    const ScanKArgs &p, uint32_t *__restrict__ flags, float *__restrict__ agg,
    uint64_t *__restrict__ incl, uint32_t epoch,
    WsHeader *hdr, int64_t seg, int64_t g, int w, int lane, float (*s_agg)[kAggFields][kWave],
    float (*s_part)[kAggFields][kWave], float (*s_bc)[kSegT][kMaxN], float (*s_A)[kWave],
    volatile uint32_t *s_timeout)
{
    float(*s_hin)[kWave] = reinterpret_cast<float(*)[kWave]>(&s_bc[0][0][0]);
    const ScanWsLayout &lay = p.lay;
    const int64_t G = lay.groups;
    const int64_t item = seg * G + g;
    const int64_t b = g / lay.n_dtiles;
    const int64_t dtile = g - b * lay.n_dtiles;
    const int64_t d = dtile * kWave + lane;
    const bool active = d < p.D;
    const int64_t dc = active ? d : (p.D - 1);  // inactive lanes read a valid row
    const int64_t t0 = seg * kSegT + (int64_t)w * kChunkT;
    // Scan-order length: L forward; in reverse L rounded up to whole chunks,
    // with the padding (identity steps) first, so that reverse chunks cover
    // the same memory runs of 32 steps as forward ones.
    const int64_t Ls = REV ? (p.L + kChunkT - 1) / kChunkT * kChunkT : p.L;
    const int nt =
        __builtin_amdgcn_readfirstlane((int)max((int64_t)0, min((int64_t)kChunkT, Ls - t0)));
    // The chunk's steps sit in kChunkT slots of one run of memory starting at
    // position p0: slot = step - t0 forward; in reverse the run ends at the
    // chunk's first step, slot = kChunkT-1 - (step - t0).  Only slots in
    // [0, khi) lie inside the sequence; the others are never read or written
    // (inputs there are the identity padding).
    const int64_t p0 = REV ? Ls - t0 - kChunkT : t0;
    const int khi = __builtin_amdgcn_readfirstlane(
        REV ? (nt > 0 ? (int)min((int64_t)kChunkT, p.L - p0) : 0) : nt);
    const int klo = 0;
    const bool vec = FULL || (p.vec && khi == kChunkT);
    const int64_t row_off = (b * p.D + dc) * p.L + p0;
    const int64_t chunk_slot = REV ? Ls / kChunkT - 1 - t0 / kChunkT : t0 / kChunkT;
    auto slot = [](int j) { return REV ? kChunkT - 1 - j : j; };

    // per-channel constants.  Loaded unconditionally (an absent dt_bias or D
    // is read through A, which has at least D entries, and ignored), so the
    // loads travel with the chunk's instead of each waiting at a branch.
    const float bias_raw = (p.dt_bias ? p.dt_bias : p.A)[dc];
    const float skip_raw = (p.Dskip ? p.Dskip : p.A)[dc];
    const float bias2 = (p.dt_bias ? bias_raw : 0.f) * kLog2e;
    const float Dd = p.Dskip ? skip_raw : 0.f;
    // General path: the A rows of the tile's channels wait in LDS (s_A[n][lane]),
    // which keeps that path within the structured path's register budget.
    // Their reciprocals (0 for A_n = 0) sit in s_part's first slot during the
    // chunk scan: s_part is first written after the barrier that ends it.
    const ARow Ar{s_A, lane};
    const ARow Ainv{s_part[0], lane};
    float a0 = -1.f, inva0 = -1.f;
    if constexpr (STRUCT) {
        a0 = p.A[dc * p.N];
        inva0 = 1.0f / a0;
    } else {
        // rows n = w + 4k of the tile's channels (this lane's channel), loads first
        constexpr int kRows = kMaxN / kWavesPerSeg;
        const int64_t dd = min(dtile * kWave + lane, p.D - 1);
        float an[kRows];
#pragma unroll
        for (int k = 0; k < kRows; ++k)
            an[k] = p.A[dd * p.N + min(w + kWavesPerSeg * k, p.N - 1)];
#pragma unroll
        for (int k = 0; k < kRows; ++k) {
            const int n = w + kWavesPerSeg * k;
            const float v = n < p.N ? an[k] : -1.f;
            s_A[n][lane] = v;
            s_part[0][n][lane] = v != 0.f ? hw_rcp(v) : 0.f;
        }
    }

    // ---- 1. local scan of this wave's chunk from a zero state -------------
    float yl[kChunkT], er[kChunkT];
    float hs[kMaxN];
    float summ;
    {
        // the small loads first (conv taps, B/C rows of a whole fp32 segment),
        // then the chunk's x and dt: a wait for the early ones then leaves the
        // chunk's loads in flight
        ConvPre<BF16> cpre;
        if constexpr (CONV)
            cpre.load(p, b * p.D + dc, dc, t0, row_off);
        constexpr bool kBcPre = FULL && !BF16;
        BcPre<STRUCT, REV, ADJ> bpre;
        if constexpr (kBcPre)
            bpre.load(p, b, seg, Ls, w * kWave + lane);
        InChunk<BF16> xin, din;
        xin.load(p.x, row_off, klo, khi, vec, 0.f);
        din.load(p.dt, row_off, klo, khi, vec, -__builtin_huge_valf());
        if constexpr (kBcPre)
            bpre.store(s_bc, w * kWave + lane);
        float xc[kChunkT];  // scan inputs of the fused front end (CONV only)
        if constexpr (CONV)
            conv_chunk<BF16>(p, cpre, xin, nt, xc);
        // adjoint scan: the input is dy = dout * SiLU(z) (x holds dout)
        InChunk<BF16> zadj;
        if (ADJ && p.z)
            zadj.load(p.z, row_off, klo, khi, vec, 0.f);
        auto xget = [&](int j) -> float {
            if constexpr (CONV)
                return xc[j];
            else if constexpr (ADJ)
                return p.z ? xin.get(slot(j)) * silu_hw(zadj.get(slot(j))) : xin.get(slot(j));
            else
                return xin.get(slot(j));
        };
        if constexpr (!kBcPre)
            stage_bc<BF16, STRUCT, REV, ADJ>(p, s_bc, b, seg, Ls, w * kWave + lane);
        __syncthreads();
        // Step values of the whole chunk first (independent chains, out of
        // the serial loop): er[j] = Δ_j A_0 / ln2, the exponent of the step's
        // decay (structured), or Δ_j/ln2.  Padded steps (dt = -inf) give Δ = 0:
        // decay 1.
#pragma unroll
        for (int j = 0; j < kChunkT; ++j) {
            const float l = softplus_log2(fmaf(din.get(slot(j)), kLog2e, bias2));  // Δ/ln2
            er[j] = STRUCT ? a0 * l : l;
        }
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            hs[n] = 0.f;
        float cumW = 0.f, cumL = 0.f;  // structured: Σ Δ A_0 / ln2; general: Σ Δ / ln2
        // structured path: the step's B row is read from LDS one step ahead,
        // into the registers the previous row has just freed, so its latency
        // hides behind the previous step's readout
        float Bc[kMaxN];
        if constexpr (STRUCT)
            lds_row(s_bc[0][w * kChunkT], Bc);
#pragma unroll
        for (int j = 0; j < kChunkT; ++j) {
            // structured: the step's decay e = exp(Δ A_0) and e - 1, from the
            // exponent w = Δ A_0 / ln2 kept in er[j]
            float ej = 0.f, emj = 0.f;
            if constexpr (STRUCT) {
                step_decay(er[j], ej, emj);
                cumW += er[j];
            }
            if (j < nt) {  // one basic block per step
                const float xv = xget(j);
                const float *Bj = s_bc[0][w * kChunkT + j];  // B (LDS broadcast)
                const float *Cj = s_bc[1][w * kChunkT + j];  // C/(n+1), or C
                float acc = 0.f;
                if constexpr (ADJ) {
                    // adjoint ν <- e_n (ν + C_n dy) (C in the first LDS matrix),
                    // unscaled; structured: e_n (ν + C dy) = s + (e_n - 1) s
                    if constexpr (STRUCT) {
                        const float e1 = ej;
                        const float em0 = emj;
                        float em = em0;
#pragma unroll
                        for (int n = 0; n < kMaxN; ++n) {
                            if (n)
                                em = fmaf(e1, em, em0);
                            const float sn = fmaf(Bc[n], xv, hs[n]);
                            hs[n] = fmaf(em, sn, sn);
                        }
                        if (j + 1 < kChunkT)
                            lds_row(s_bc[0][w * kChunkT + j + 1], Bc);
                    } else {
                        const float l = er[j];
                        cumL += l;
#pragma unroll
                        for (int n = 0; n < kMaxN; ++n)
                            hs[n] = hw_exp2(Ar[n] * l) * fmaf(Bj[n], xv, hs[n]);
                    }
                } else if constexpr (STRUCT) {
                    // ĥ <- ĥ + (e_n - 1)(ĥ + B_n x), with e_n - 1 = e^(n+1) - 1
                    // built as (e_n - 1) = e (e_(n-1) - 1) + (e - 1)
                    float Cr[kMaxN];
                    lds_row(Cj, Cr);
                    const float e1 = ej;
                    const float em0 = emj;
                    float em = em0;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        if (n)
                            em = fmaf(e1, em, em0);
                        const float sn = fmaf(Bc[n], xv, hs[n]);
                        hs[n] = fmaf(em, sn, hs[n]);
                    }
                    if (j + 1 < kChunkT)
                        lds_row(s_bc[0][w * kChunkT + j + 1], Bc);
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n)
                        acc = fmaf(Cr[n], hs[n], acc);
                    yl[j] = fmaf(acc, inva0, Dd * xv);
                } else {
                    const float l = er[j];
                    const float delta = l * kLn2;
                    cumL += l;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        const float wn = Ar[n] * l;
                        const float en = hw_exp2(wn);  // exp(Δ A_n); 1 when A_n = 0
                        const float coef = zoh_coef_w(wn, delta, en, Ainv[n]);
                        hs[n] = fmaf(en, hs[n], coef * (Bj[n] * xv));
                        acc = fmaf(Cj[n], hs[n], acc);
                    }
                    yl[j] = fmaf(Dd, xv, acc);
                    er[j] = cumL;
                }
            }
            // structured forward: er[j] becomes the cumulative decay E_j since
            // the chunk's start (a padding step adds 0 to the exponent).  It is
            // 2^(Σ w), not a product of the steps' decays: those sit within a
            // few ulp of 1 when Δ A_0 is small, and a product of many of them,
            // raised to the power n+1 by the fix-up, loses about (n+1) ulp per
            // step (the products had put the outputs of a 4096-step fp32 scan
            // with Δ near 1e-5 and an initial state 1.4e-3 off)
            if constexpr (STRUCT && !ADJ)
                er[j] = hw_exp2(cumW);
        }
        if constexpr (STRUCT) {
            summ = cumW;  // the chunk's decay, as its exponent sum
            // back to true units: h_n = ĥ_n / A_n (the adjoint is unscaled)
            if constexpr (!ADJ) {
#pragma unroll
                for (int n = 0; n < kMaxN; ++n)
                    hs[n] = hs[n] * (inva0 / (float)(n + 1));
            }
        } else {
            summ = cumL;
        }
    }

    // z is only needed by the final gating.  bf16 z (16 VGPRs) is requested
    // now, so it arrives while the workgroup resolves its start state; wave 0
    // first publishes its record (that publish waits for every outstanding
    // memory operation of the wave).  fp32 z (32 VGPRs) is requested once the
    // start state is known, ahead of the fix-up.
    InChunk<BF16> zin;
    if (BF16 && !ADJ && p.y && p.z && w != 0)
        zin.load(p.z, row_off, klo, khi, vec, 0.f);

    // ---- 2. combine chunk maps inside the workgroup ------------------------
    s_agg[w][0][lane] = summ;
#pragma unroll
    for (int n = 0; n < kMaxN; ++n)
        s_agg[w][1 + n][lane] = hs[n];
    __syncthreads();
    // ---- 3. segment map and the records this segment folds ------------------
    // Fixed association order, independent of scheduling: a segment folds the
    // aggregates of the earlier segments of its superblock, in order, onto the
    // inclusive state that ends the previous superblock (-1 = h0).
    const int64_t SB = lay.superseg;
    const bool chain = SB == 1;  // each segment takes its predecessor's end state
    const int64_t sI = (seg / SB) * SB - 1;
    const int64_t depth = seg - 1 - sI;
    // Step-4 partials of waves 1..3: waves 1, 2 in s_part[1], s_part[2]; the
    // last wave's in s_agg's last slot, which nothing reads after step 3 (the
    // per-wave start states of step 6 only apply the maps of earlier chunks).
    auto partial_slot = [&](int k) -> float(*)[kWave] {
        return k == kWavesPerSeg - 1 ? s_agg[kWavesPerSeg - 1] : s_part[k];
    };
    if (w == 0) {
        float F = s_agg[0][0][lane];
        float Sg[kMaxN];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            Sg[n] = s_agg[0][1 + n][lane];
#pragma unroll
        for (int k = 1; k < kWavesPerSeg; ++k) {
            const float fk = s_agg[k][0][lane];
            apply_map<STRUCT>(fk, [&](int n) { return s_agg[k][1 + n][lane]; }, Ar, Sg);
            F = combine_summary(F, fk);
        }
        // the segment map, for step 5 (slot 0 of s_part; wave 0 keeps its own
        // step-4 partial in registers)
        s_part[0][0][lane] = F;
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            s_part[0][1 + n][lane] = Sg[n];
        if (seg + 1 < lay.n_seg && !chain) {
            // successors in this superblock fold this segment's aggregate
            float *rec = agg + item * (kAggFields * kWave);
            store_rec(rec + lane, F);
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                store_rec(rec + (1 + n) * kWave + lane, Sg[n]);
            publish_flag(flags + item, kFlagAgg, lane);
        }
        if (BF16 && !ADJ && p.y && p.z)
            zin.load(p.z, row_off, klo, khi, vec, 0.f);
        if (depth > 0) {
            // wait for the aggregates this segment folds: lane j < depth
            // watches segment seg-1-j (the inclusive state of sI is awaited
            // later, after the fold, so that the superblock-to-superblock chain
            // only carries one map application per hop)
            const bool ok = wait_flags(flags + (seg - 1 - lane) * G + g,
                                       lane < depth ? kFlagAgg : 0u, hdr, lane, p.spin_limit);
            if (!ok && lane == 0)
                *s_timeout = 1u;
        }
    }
    __syncthreads();
    // ---- 4. fold the predecessors' aggregates, four waves in parallel --------
    {
        const int64_t per = (depth + kWavesPerSeg - 1) / kWavesPerSeg;
        const int64_t lo = min(depth, (int64_t)w * per), hi = min(depth, lo + per);
        float pf = 0.f;  // identity map
        float ps[kMaxN];
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            ps[n] = 0.f;
        for (int64_t j = lo; j < hi; j += 2) {  // records in time order, two per round trip
            const bool two = j + 1 < hi;
            const float *r0 = agg + ((sI + 1 + j) * G + g) * (kAggFields * kWave);
            const float *r1 = two ? r0 + G * (kAggFields * kWave) : r0;
            float v0[kAggFields], v1[kAggFields];
#pragma unroll
            for (int k = 0; k < kAggFields; ++k) {
                v0[k] = load_rec(r0 + k * kWave + lane);
                v1[k] = load_rec(r1 + k * kWave + lane);
            }
            apply_map<STRUCT>(v0[0], [&](int n) { return v0[1 + n]; }, Ar, ps);
            pf = combine_summary(pf, v0[0]);
            if (two) {
                apply_map<STRUCT>(v1[0], [&](int n) { return v1[1 + n]; }, Ar, ps);
                pf = combine_summary(pf, v1[0]);
            }
        }
        if (w != 0) {
            float(*slot)[kWave] = partial_slot(w);
            slot[0][lane] = pf;
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                slot[1 + n][lane] = ps[n];
        }
        __syncthreads();
        // ---- 5. segment start state and inclusive record ---------------------
        if (w == 0) {
            float hin[kMaxN];
            if (sI < 0) {
#pragma unroll
                for (int n = 0; n < kMaxN; ++n)
                    hin[n] = (p.h0 && n < p.N) ? p.h0[(b * p.D + dc) * p.N + n] : 0.f;
            } else if (chain) {
                // the previous segment's end state: its flag, then its record
                const bool ok = wait_flags(flags + sI * G + g, lane == 0 ? kFlagAgg : 0u, hdr,
                                           lane, p.spin_limit);
                if (!ok && lane == 0)
                    *s_timeout = 1u;
                const float *rec = agg + (sI * G + g) * (kAggFields * kWave) + lane;
#pragma unroll
                for (int n = 0; n < kMaxN; ++n)
                    hin[n] = load_rec(rec + (1 + n) * kWave);
            } else {
                // the previous superblock's end state: poll its tagged record
                const uint64_t *rec =
                    incl + ((sI / SB) * G + g) * (kInclFields * kWave) + lane;
                for (int spins = 0;; ++spins) {
                    bool ok = true;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        const uint64_t wd = load_tagged(rec + n * kWave);
                        hin[n] = __uint_as_float((uint32_t)wd);
                        ok = ok & ((uint32_t)(wd >> 32) == epoch);
                    }
                    if (__ballot(!ok) == 0ull)
                        break;
                    if (spins >= p.spin_limit) {  // not expected with the default limit
                        if (lane == 0)
                            atomicOr(&hdr->error, kErrSpinTimeout);
                        if (lane == 0)
                            *s_timeout = 1u;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            // a carry wait that gave up: this segment's start state (and so its
            // outputs, its end state and every later segment's) is NaN
            if (*s_timeout) {
#pragma unroll
                for (int n = 0; n < kMaxN; ++n)
                    hin[n] = __builtin_nanf("");
            }
            // wave 0's own partial is still in registers; then waves 1..3
            apply_map<STRUCT>(pf, [&](int n) { return ps[n]; }, Ar, hin);
#pragma unroll
            for (int k = 1; k < kWavesPerSeg; ++k) {
                float(*slot)[kWave] = partial_slot(k);
                apply_map<STRUCT>(slot[0][lane], [&](int n) { return slot[1 + n][lane]; }, Ar,
                                  hin);
            }
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                s_hin[n][lane] = hin[n];
            const bool publish = seg + 1 < lay.n_seg && (seg + 1) % SB == 0;
            const bool last = seg + 1 == lay.n_seg;
            if (publish || (last && p.h_last)) {
                // state at the end of the segment
                apply_map<STRUCT>(s_part[0][0][lane],
                                  [&](int n) { return s_part[0][1 + n][lane]; }, Ar, hin);
                if (publish && chain) {
                    // in the segment's own record slot, then its flag
                    float *rec = agg + item * (kAggFields * kWave) + lane;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n)
                        store_rec(rec + (1 + n) * kWave, hin[n]);
                    publish_flag(flags + item, kFlagAgg, lane);
                } else if (publish) {
                    uint64_t *rec =
                        incl + ((seg / SB) * G + g) * (kInclFields * kWave) + lane;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n)
                        store_tagged(rec + n * kWave, hin[n], epoch);
                } else if (active) {
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n)
                        if (n < p.N)
                            p.h_last[(b * p.D + d) * p.N + n] = hin[n];
                }
            }
        }
    }
    __syncthreads();

    if (nt <= 0)
        return;

    // ---- 6. this wave's start state, fix-up, gate, store -------------------
    float hin[kMaxN];
#pragma unroll
    for (int n = 0; n < kMaxN; ++n)
        hin[n] = s_hin[n][lane];
    for (int k = 0; k < w; ++k)
        apply_map<STRUCT>(s_agg[k][0][lane], [&](int n) { return s_agg[k][1 + n][lane]; }, Ar,
                          hin);
    if (p.chunk_states) {
        // the chunk's start state, for the backward pass ([group][slot][n][lane])
        float *cs = p.chunk_states + ((g * p.n_cslots + chunk_slot) * kMaxN) * kWave + lane;
#pragma unroll
        for (int n = 0; n < kMaxN; ++n)
            cs[n * kWave] = hin[n];
    }
    if (ADJ || p.y == nullptr)
        return;
    if (!BF16 && p.z)
        zin.load(p.z, row_off, klo, khi, vec, 0.f);
    const bool zero_start = (seg == 0 && w == 0 && p.h0 == nullptr);
    // The step conditions of the fix-up loops must not be shared with the scan
    // loops (keeping 32 condition masks alive costs scalar registers): give the
    // compiler a copy of nt it cannot prove equal.
    int ntf = nt;
    __asm__ volatile("" : "+s"(ntf));

    if (!zero_start) {
        if constexpr (STRUCT) {
            // coefficient of the carried state in scaled units: (n+1) A_0 h_in,n
            float hsc[kMaxN];
#pragma unroll
            for (int n = 0; n < kMaxN; ++n)
                hsc[n] = (a0 * (float)(n + 1)) * hin[n];
#pragma unroll
            for (int j = 0; j < kChunkT; ++j) {
                if (j < ntf) {
                    const float *cs = s_bc[1][w * kChunkT + j];  // C/(n+1)
                    const float Ej = er[j];
                    // Horner from the last state (starting from 0 would cost an
                    // fma with 0, which the compiler keeps)
                    float qh = cs[kMaxN - 1] * hsc[kMaxN - 1];
#pragma unroll
                    for (int n = kMaxN - 2; n >= 0; --n)
                        qh = fmaf(qh, Ej, cs[n] * hsc[n]);
                    yl[j] = fmaf(qh * Ej, inva0, yl[j]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kChunkT; ++j) {
                if (j < ntf) {
                    const float *cr = s_bc[1][w * kChunkT + j];  // C
                    // cumulative Δ/ln2, kept finite so that A_n = 0 gives 2^0 = 1
                    const float Lj = fminf(er[j], __FLT_MAX__);
                    float corr = 0.f;
#pragma unroll
                    for (int n = 0; n < kMaxN; ++n) {
                        const float gdec = hw_exp2(Ar[n] * Lj);
                        corr = fmaf(cr[n] * gdec, hin[n], corr);
                    }
                    yl[j] += corr;
                }
            }
        }
    }
    if (p.z) {
#pragma unroll
        for (int j = 0; j < kChunkT; ++j) {
            yl[j] *= silu_hw(zin.get(slot(j)));
        }
    }
    if (active)
        store_chunk<BF16>(p.y, row_off, klo, khi, vec, p.accumulate != 0,
                          [&](int k) { return yl[slot(k)]; });
}

// FULL: every chunk of the problem is whole and its rows are 16-byte aligned
// (L a multiple of kSegT, aligned x, dt, z, y; N = 16 with aligned B, C), so
// the inputs take 128-bit loads with no bounds checks and B/C go through
// registers ahead of the chunk's own loads.
template <bool BF16, bool CONV, bool REV, bool ADJ, bool FULL>
__global__ void __launch_bounds__(kWave *kWavesPerSeg, kScanWavesPerSimd) scan_main_kernel(
    ScanKArgs p, const uint32_t *__restrict__ tiles)
{
    __shared__ float s_agg[kWavesPerSeg][kAggFields][kWave];
    __shared__ float s_part[kWavesPerSeg - 1][kAggFields][kWave];
    __shared__ float s_A[kMaxN][kWave];  // general path: A of the tile's channels
    // B and C (C/(n+1) on the structured path) of the segment's steps; once
    // every wave has finished its chunk scan the B half holds the start states
    __shared__ __attribute__((aligned(16))) float s_bc[2][kSegT][kMaxN];
    __shared__ uint32_t s_ticket;
    __shared__ uint32_t s_timeout;  // a carry wait of this workgroup gave up

    WsHeader *hdr = reinterpret_cast<WsHeader *>(p.ws + p.lay.off_header);
    uint32_t *flags = reinterpret_cast<uint32_t *>(p.ws + p.lay.off_flags);
    float *agg = reinterpret_cast<float *>(p.ws + p.lay.off_agg);
    uint64_t *incl = reinterpret_cast<uint64_t *>(p.ws + p.lay.off_incl);
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(hdr->epoch);

    if (threadIdx.x == 0) {
        s_ticket = atomicAdd(&hdr->ticket, 1u);
        s_timeout = 0u;
    }
    __syncthreads();
    const int64_t item = (int64_t)__builtin_amdgcn_readfirstlane(s_ticket);
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int64_t seg = item / p.lay.groups;
    const int64_t g = item - seg * p.lay.groups;
    const int64_t dtile = g % p.lay.n_dtiles;
    const uint32_t path = __builtin_amdgcn_readfirstlane(tiles[dtile]);
    if (path == kPathStructured)
        scan_segment<BF16, true, CONV, REV, ADJ, FULL>(p, flags, agg, incl, epoch, hdr, seg, g, w, lane, s_agg,
                                       s_part, s_bc, s_A, &s_timeout);
    else
        scan_segment<BF16, false, CONV, REV, ADJ, FULL>(p, flags, agg, incl, epoch, hdr, seg, g, w, lane, s_agg,
                                        s_part, s_bc, s_A, &s_timeout);
}

// Writes h_last = h0 (or zeros) for an empty sequence (L == 0).
__global__ void copy_or_zero_kernel(const float *__restrict__ src, float *__restrict__ dst,
                                    int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        dst[i] = src ? src[i] : 0.f;
}

// Raw inputs a later call continues from: the last K-1 steps of the sequence
// with the carried-in ones in front, state_out[s] = x_ext[L + s] where
// x_ext[t] = x[t] for t >= 0 and state_in[K-1+t] (or 0) for t < 0.  One
// thread per channel, slots in increasing order, so state_out may be the same
// buffer as state_in (slot s reads slot L+s >= s before slot s is written).
template <typename T>
__global__ void conv_state_kernel(const T *__restrict__ x, const T *state_in, T *state_out,
                                  int64_t BD, int64_t L, int K)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= BD)
        return;
    for (int s = 0; s < K - 1; ++s) {
        const int64_t t = L - (K - 1) + s;
        T v = T(0);
        if (t >= 0)
            v = x[i * L + t];
        else if (state_in)
            v = state_in[i * (K - 1) + (K - 1) + t];
        state_out[i * (K - 1) + s] = v;
    }
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
    l.off_agg = off;
    off = round_up(off + (size_t)l.n_items * kAggFields * kWave * 4, 256);
    l.superseg = l.groups >= kChainGroups ? 1 : kSuperSeg;
    l.off_incl = off;  // superblocks: one tagged record per superblock and group
    if (l.superseg > 1)
        off = round_up(off + (size_t)(((l.n_seg + l.superseg - 1) / l.superseg) * l.groups) *
                                 kInclFields * kWave * 8,
                       256);
    l.total = off;
    return l;
}

hipError_t launch_selective_scan(const ScanArgs &a, hipStream_t s)
{
    const ScanWsLayout &lay = a.lay;
    const int64_t BD = a.B * a.D;
    auto conv_state = [&]() -> hipError_t {
        if (!a.conv_K || !a.conv_state_out || a.conv_K < 2 || BD == 0)
            return hipSuccess;
        const dim3 grid((unsigned)((BD + 255) / 256));
        if (a.bf16)
            hipLaunchKernelGGL(conv_state_kernel<uint16_t>, grid, dim3(256), 0, s,
                               (const uint16_t *)a.x, (const uint16_t *)a.conv_state_in,
                               (uint16_t *)a.conv_state_out, BD, a.L, a.conv_K);
        else
            hipLaunchKernelGGL(conv_state_kernel<float>, grid, dim3(256), 0, s,
                               (const float *)a.x, (const float *)a.conv_state_in,
                               (float *)a.conv_state_out, BD, a.L, a.conv_K);
        return hipGetLastError();
    };
    if (a.L == 0) {
        if (a.h_last) {
            const int64_t n = a.B * a.D * a.N;
            hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)),
                               dim3(256), 0, s, a.h0, a.h_last, n);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        return conv_state();
    }
    if (lay.n_items == 0)
        return hipSuccess;
    // prep: flags and header, then tile classification, then the tags of the
    // inclusive records (every superblock but the last is polled), each part
    // from a wave boundary
    const int64_t n_flags = lay.n_items;
    const int64_t classify_base = (n_flags + kWave - 1) / kWave * kWave;
    const int64_t clear_base = classify_base + lay.n_dtiles * kWave;
    const int64_t n_sb = (lay.n_seg + lay.superseg - 1) / lay.superseg;
    const int64_t n_clear16 =
        lay.superseg > 1 ? (n_sb - 1) * lay.groups * kInclFields * kWave * 8 / 16 : 0;
    const int64_t total = clear_base + n_clear16;
    hipLaunchKernelGGL(scan_prep_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       a.A, a.ws, lay, a.D, a.N, n_flags, classify_base, clear_base, n_clear16,
                       a.keep_error ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;

    ScanKArgs k;
    k.x = a.x;
    k.dt = a.dt;
    k.z = a.z;
    k.Bm = a.Bm;
    k.Cm = a.Cm;
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
    k.conv_w = a.conv_w;
    k.conv_b = a.conv_b;
    k.conv_state_in = a.conv_state_in;
    k.conv_K = a.conv_K;
    k.accumulate = a.accumulate ? 1 : 0;
    k.chunk_states = a.chunk_states;
    k.n_cslots = lay.n_seg * kWavesPerSeg;
    k.spin_limit = a.spin_limit;
    const size_t esz = a.bf16 ? 2 : 4;
    const uintptr_t amask = (uintptr_t)a.x | (uintptr_t)a.dt | (uintptr_t)a.y |
                            (uintptr_t)(a.z ? a.z : a.x);
    k.vec = ((amask & 15u) == 0 && ((size_t)a.L * esz) % 16 == 0) ? 1 : 0;
    k.bc_vec = (a.N == kMaxN && (((uintptr_t)a.Bm | (uintptr_t)a.Cm) & 15u) == 0) ? 1 : 0;
    const uint32_t *tiles = reinterpret_cast<const uint32_t *>(a.ws + lay.off_tiles);
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, s);
    const dim3 grid((unsigned)lay.n_items), block(kWave * kWavesPerSeg);
    // fp32 problems of whole segments with aligned rows take the FULL kernel
    // (no ragged chunk, so no branch around any input load); bf16 ones do not
    // need it (their loads already leave together) and would spill with it
    const bool full = !a.bf16 && k.vec && k.bc_vec && a.L % kSegT == 0;
#define MAMBA_SCAN_LAUNCH(BF, CV, RV, AJ, FL) \
    hipLaunchKernelGGL((scan_main_kernel<BF, CV, RV, AJ, FL>), grid, block, 0, s, k, tiles)
#define MAMBA_SCAN_LAUNCH_F32(CV, RV, AJ)                 \
    do {                                                  \
        if (full)                                         \
            MAMBA_SCAN_LAUNCH(false, CV, RV, AJ, true);   \
        else                                              \
            MAMBA_SCAN_LAUNCH(false, CV, RV, AJ, false);  \
    } while (0)
    if (a.bf16) {
        if (a.conv_K)
            MAMBA_SCAN_LAUNCH(true, true, false, false, false);
        else if (a.adjoint)
            MAMBA_SCAN_LAUNCH(true, false, true, true, false);
        else if (a.reverse)
            MAMBA_SCAN_LAUNCH(true, false, true, false, false);
        else
            MAMBA_SCAN_LAUNCH(true, false, false, false, false);
    } else {
        if (a.conv_K)
            MAMBA_SCAN_LAUNCH_F32(true, false, false);
        else if (a.adjoint)
            MAMBA_SCAN_LAUNCH_F32(false, true, true);
        else if (a.reverse)
            MAMBA_SCAN_LAUNCH_F32(false, true, false);
        else
            MAMBA_SCAN_LAUNCH_F32(false, false, false);
    }
#undef MAMBA_SCAN_LAUNCH_F32
#undef MAMBA_SCAN_LAUNCH
    e = hipGetLastError();
    if (a.ev_stop)
        (void)hipEventRecord(a.ev_stop, s);
    if (e != hipSuccess)
        return e;
    return conv_state();
}

}  // namespace mamba
