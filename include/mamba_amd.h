/*
 * mamba_amd.h -- C ABI of the MI355X (gfx950) selective state-space library.
 *
 * Three operations make up the data-parallel hot path of a Mamba block:
 *   mamba_conv1d_silu            causal depthwise conv1d + SiLU front end
 *   mamba_selective_scan_fwd     fused selective-scan forward (prefill)
 *   mamba_selective_state_update single-token recurrent step (decode)
 * the scan with direction / accumulate flags (mamba_selective_scan_fwd_ex),
 * and three that join the front end to the scan:
 *   mamba_conv1d_selective_scan_fwd      conv1d + SiLU fused into the scan
 *   mamba_conv1d_update                  single-token conv step with its state
 *   mamba_conv1d_selective_state_update  that conv step and the decode step fused
 * the scan's backward pass (mamba_selective_scan_bwd), the Mamba-2 form of
 * the scan on the matrix cores (mamba_ssd_scan_fwd),
 * plus workspace sizing and status helpers.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller, contiguous,
 *     row-major in the layout stated at the call; the library never frees or
 *     keeps it.  Optional inputs may be NULL where stated.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream).  They allocate no memory.
 *   - Arguments are validated on the host before any HIP call; on a bad
 *     argument the call returns a status other than MAMBA_OK and launches
 *     nothing.  A failure to launch returns MAMBA_ERR_LAUNCH.  Faults inside a
 *     kernel surface at the caller's next synchronisation, as usual for HIP.
 *   - Outputs must not overlap inputs (only the decode state is in/out).
 *   - Sizes: each of B, D, L (or H, P) and the product of the non-zero ones
 *     is at most 2^40, and each call's launch grids must fit one launch:
 *     about 2^31 channels for the decode calls (B*D), 2^31 threads for the
 *     standalone conv (B*D*ceil(L/4)), 2^23 64-channel x 128-step segments for
 *     the scans (2^21 for the backward, with B*L < 2^25), B*H < 2^24 for the
 *     Mamba-2 form.  Beyond them a call returns MAMBA_ERR_SHAPE.
 *   - Element types: MAMBA_F32 = float, MAMBA_BF16 = bfloat16 (stored as
 *     uint16, round-to-nearest-even on output).  Parameters (A, dt_bias, D,
 *     conv weights, states) are always float.
 *   - Arithmetic is fp32 throughout, including the recurrent state.
 *   - Thread safety: calls may be issued from several host threads; calls
 *     that share a workspace must be ordered on one stream.
 *
 * Notation: B batch, D channels (d_inner), L sequence length, N state size
 * (1..16), K conv taps.  The model is the selective SSM of the Mamba papers:
 *   Δ_t   = softplus(dt_t + dt_bias)                       (input-dependent step)
 *   Ā_t   = exp(Δ_t A),  B̄_t = (Δ_t A)^-1 (exp(Δ_t A) - I) Δ_t B_t   (zero-order hold)
 *   h_t   = Ā_t h_{t-1} + B̄_t x_t,   y_t = <C_t, h_t> + D x_t
 *   out_t = y_t * SiLU(z_t)
 * with A diagonal (one value per channel d and state n).
 */
#ifndef MAMBA_AMD_H
#define MAMBA_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_AMD_ABI_VERSION 9
#define MAMBA_MAX_STATE 16
#define MAMBA_MAX_CONV_TAPS 8
#define MAMBA_MAX_FUSED_CONV_TAPS 4
/* Scratch that mamba_selective_scan_fwd_noalloc uses in place of a workspace. */
#define MAMBA_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum { MAMBA_F32 = 0, MAMBA_BF16 = 1 } mamba_dtype;

typedef enum {
    MAMBA_OK = 0,
    MAMBA_ERR_NULL = 1,        /* a required pointer is NULL                  */
    MAMBA_ERR_SHAPE = 2,       /* a size is negative or the product too large */
    MAMBA_ERR_DTYPE = 3,       /* dtype is not MAMBA_F32 / MAMBA_BF16         */
    MAMBA_ERR_UNSUPPORTED = 4, /* N outside 1..16, K outside 1..8             */
    MAMBA_ERR_ALIGN = 5,       /* pointer not aligned to its element size     */
    MAMBA_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
    MAMBA_ERR_WORKSPACE = 7,   /* workspace missing, misaligned or too small  */
    MAMBA_ERR_LAUNCH = 8,      /* HIP reported an error when launching        */
    MAMBA_ERR_DEVICE = 9,      /* no HIP device, or not a gfx950 device       */
    MAMBA_ERR_TIMEOUT = 10     /* a scan's carry wait gave up (see below)     */
} mamba_status;

/* Static, human-readable name of a status value (never NULL). */
const char *mamba_status_string(int status);

/* MAMBA_AMD_ABI_VERSION of the compiled library. */
int mamba_abi_version(void);

/*
 * Causal depthwise conv1d over time, then SiLU (the block's front end:
 * "Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式", §3.1, causal
 * Conv1D before the selective SSM; kernel size d_conv = 4 in
 * "Mamba架构与SSM模型：高效序列建模技术解析", §3.2):
 *   out[b,d,t] = SiLU( bias[d] + sum_{k<K} w[d,k] * x[b,d,t-(K-1)+k] ),  x[t<0] = 0.
 *   x, out : [B, D, L] of `dtype`;  w : [D, K] float;  bias : [D] float or NULL.
 * out must not overlap x.  K in 1..8.  MAMBA_ERR_SHAPE also when
 * B * D * ceil(L / 4) >= 2^31 (one launch covers the whole problem).
 */
mamba_status mamba_conv1d_silu(const void *x, const float *w, const float *bias, void *out,
                               int64_t B, int64_t D, int64_t L, int64_t K, mamba_dtype dtype,
                               void *stream);

/*
 * Bytes of device workspace mamba_selective_scan_fwd needs for this shape
 * (0 only for an empty problem).  The workspace is scratch owned by the
 * caller: it needs no initialisation, holds nothing between calls, and must
 * be 256-byte aligned.
 */
size_t mamba_selective_scan_fwd_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                               mamba_dtype io);

/*
 * Fused selective-scan forward: softplus step, zero-order-hold discretisation
 * ("Mamba架构与SSM模型：高效序列建模技术解析", §2.1-2.2), the selective
 * recurrence with readout after the update ("Mamba状态空间模型深度解析：
 * 挑战Transformer的下一代序列建模范式", §2.1), the D skip and the SiLU(z) gate
 * (same page, §3.1), for every (b, d) sequence, in one pass over the inputs.
 * Long sequences are cut into chunks whose end states are carried across
 * chunks ("Mamba: Linear-Time Sequence Modeling with Selective SSMs", section
 * on the block-wise selective scan with a prefix state passed forward).
 *
 *   x, dt, z, y : [B, D, L] of `io`            (z NULL = no gate)
 *   dt_bias     : [D] float or NULL (= 0)      Dskip : [D] float or NULL (= 0)
 *   A           : [D, N] float (diagonal state matrix, one row per channel)
 *   Bm, Cm      : [B, L, N] of `io`, shared by every channel of batch b
 *   h0          : [B, D, N] float or NULL (= zero initial state)
 *   h_last      : [B, D, N] float or NULL (= not returned): state after step L-1
 *   workspace   : >= mamba_selective_scan_fwd_workspace_size(...) bytes
 * h0/h_last let a long sequence be scanned in several calls or handed to the
 * decode step.  y and h_last must not overlap any input, each other or the
 * workspace.
 */
mamba_status mamba_selective_scan_fwd(const void *x, const void *dt, const float *dt_bias,
                                      const float *A, const void *Bm, const void *Cm,
                                      const float *Dskip, const void *z, const float *h0,
                                      void *y, float *h_last, void *workspace,
                                      size_t workspace_bytes, int64_t B, int64_t D, int64_t L,
                                      int64_t N, mamba_dtype io, void *stream);

/*
 * mamba_selective_scan_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, the same arguments without the workspace.
 * The library's own scratch, MAMBA_NOALLOC_SCRATCH_BYTES (64 MiB) of device
 * memory that each GPU it runs on holds until the process ends, takes the
 * workspace's place; the call allocates nothing (no hipMalloc, no allocating
 * library routine).  Shapes whose workspace
 * (mamba_selective_scan_fwd_workspace_size) exceeds the scratch return
 * MAMBA_ERR_WORKSPACE before any HIP call: B=2 D=1536 L=8192 needs 16.5 MB and
 * B=8 D=5120 L=2048 45 MB; B=1 D=1536 L=131072 (132 MB) does not fit.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap in
 * time on one GPU (two streams, or two host threads) race and must not be
 * made; calls ordered on one stream are fine (each call initialises what it
 * reads of the scratch).  The first call on a device looks up that device's
 * copy of the scratch (MAMBA_ERR_DEVICE if that fails).
 */
mamba_status mamba_selective_scan_fwd_noalloc(const void *x, const void *dt,
                                              const float *dt_bias, const float *A,
                                              const void *Bm, const void *Cm,
                                              const float *Dskip, const void *z,
                                              const float *h0, void *y, float *h_last,
                                              int64_t B, int64_t D, int64_t L, int64_t N,
                                              mamba_dtype io, void *stream);

/*
 * Single-token decode step (the recurrent, fixed-size-state mode used at
 * inference: "Mamba架构深度剖析：如何以线性时间重塑序列建模", §3): for every
 * (b, d), one step of the recurrence above on the stored state h, updated in
 * place, and the gated output of that token.
 *   h           : [B, D, N] float, read and overwritten
 *   x, dt, z, y : [B, D] of `io`  (z NULL = no gate)
 *   Bm, Cm      : [B, N] of `io`
 *   A [D, N], dt_bias [D] or NULL, Dskip [D] or NULL : float
 *   flags       : 0, or MAMBA_STEP_STREAM_STATE
 * y must not overlap h or any input.  Unknown flags return
 * MAMBA_ERR_UNSUPPORTED.
 */
mamba_status mamba_selective_state_update(float *h, const void *x, const void *dt,
                                          const float *dt_bias, const float *A,
                                          const void *Bm, const void *Cm, const float *Dskip,
                                          const void *z, void *y, int64_t B, int64_t D,
                                          int64_t N, mamba_dtype io, unsigned flags,
                                          void *stream);

/* Flag of the decode steps (mamba_selective_state_update,
 * mamba_conv1d_selective_state_update): a cache hint only, the results are
 * the same bits.  The state h is loaded and stored with nontemporal hints, so
 * it streams through the caches instead of being kept in them.  For callers
 * whose state will not be read again before other traffic evicts it, as in a
 * model whose layers each advance their own state once per token: there it
 * raises the step's bandwidth; a state that stays cached from one call to the
 * next (the same state stepped again at once) is slower with it. */
#define MAMBA_STEP_STREAM_STATE 1u

/* Flags of mamba_selective_scan_fwd_ex. */
#define MAMBA_SCAN_REVERSE 1u    /* scan from step L-1 down to step 0 */
#define MAMBA_SCAN_ACCUMULATE 2u /* add the gated output to y instead of storing it */

/*
 * mamba_selective_scan_fwd with flags, for the scan directions of a
 * bidirectional layer ("Mamba架构与SSM模型：高效序列建模技术解析", §2: sequences
 * modelled in both directions by alternating the scan direction; §3: the
 * module's bidirectional option).
 *   MAMBA_SCAN_REVERSE     the same recurrence in reversed time: the state runs
 *                          from step L-1 down to step 0, so y_t sees steps
 *                          t..L-1.  h0 is the state before step L-1, h_last the
 *                          state after step 0.  Equal to the forward scan of the
 *                          time-reversed x, dt, z, Bm, Cm, reversed back.
 *   MAMBA_SCAN_ACCUMULATE  y[...] += out instead of y[...] = out (bf16: the sum
 *                          is formed in fp32 from the stored value and rounded
 *                          once), so a forward call followed by a reverse call
 *                          with this flag leaves (y_fwd + y_rev) in y.
 * Unknown flags return MAMBA_ERR_UNSUPPORTED.  Every other argument and rule
 * is as for mamba_selective_scan_fwd (flags = 0 is that call).
 */
mamba_status mamba_selective_scan_fwd_ex(const void *x, const void *dt, const float *dt_bias,
                                         const float *A, const void *Bm, const void *Cm,
                                         const float *Dskip, const void *z, const float *h0,
                                         void *y, float *h_last, void *workspace,
                                         size_t workspace_bytes, int64_t B, int64_t D, int64_t L,
                                         int64_t N, mamba_dtype io, unsigned flags, void *stream);

/*
 * The block's front end and the scan in one pass: the scan input is
 * SiLU(causal depthwise conv1d of x_raw) ("Mamba状态空间模型深度解析：挑战
 * Transformer的下一代序列建模范式", §3.1: causal Conv1D, then the selective
 * SSM, then the SiLU gate), computed inside the scan kernel, so the conv
 * output never goes to memory.  Same result as mamba_conv1d_silu followed by
 * mamba_selective_scan_fwd, except that the conv output is not rounded to
 * `io` in between.
 *   x_raw          : [B, D, L] of `io`
 *   conv_w         : [D, K] float, K in 1..4 (MAMBA_MAX_FUSED_CONV_TAPS)
 *   conv_bias      : [D] float or NULL (= 0)
 *   conv_state_in  : [B, D, K-1] of `io` or NULL (= zeros): raw inputs of the
 *                    K-1 steps before t = 0, oldest first
 *   conv_state_out : [B, D, K-1] of `io` or NULL (= not returned): raw inputs
 *                    of the last K-1 steps (carried-in ones when L < K-1), for
 *                    a later call or mamba_conv1d_update.  It may be the same
 *                    buffer as conv_state_in; it must not overlap anything else.
 * Every other argument is as for mamba_selective_scan_fwd (same workspace size).
 */
mamba_status mamba_conv1d_selective_scan_fwd(
    const void *x_raw, const float *conv_w, const float *conv_bias, int64_t K,
    const void *conv_state_in, void *conv_state_out, const void *dt, const float *dt_bias,
    const float *A, const void *Bm, const void *Cm, const float *Dskip, const void *z,
    const float *h0, void *y, float *h_last, void *workspace, size_t workspace_bytes, int64_t B,
    int64_t D, int64_t L, int64_t N, mamba_dtype io, void *stream);

/*
 * Decode step of the front end ("Mamba架构深度剖析：如何以线性时间重塑序列建模",
 * §3: recurrent inference with a fixed-size state; the causal conv keeps its
 * last K-1 raw inputs as state):
 *   out[b,d] = SiLU(bias[d] + sum_{k<K-1} w[d,k] state[b,d,k] + w[d,K-1] x[b,d])
 *   state[b,d,:] <- (state[b,d,1:], x[b,d])
 *   state   : [B, D, K-1] of `dtype`, read and overwritten (may be NULL when K = 1)
 *   x, out  : [B, D] of `dtype`;  w : [D, K] float;  bias : [D] float or NULL
 * K in 1..8.  out must not overlap state, x, w or bias.
 */
mamba_status mamba_conv1d_update(void *state, const void *x, const float *w, const float *bias,
                                 void *out, int64_t B, int64_t D, int64_t K, mamba_dtype dtype,
                                 void *stream);

/*
 * The block's whole decode step in one pass: the front end's decode step
 * (mamba_conv1d_update) on the raw input x_raw, whose output feeds the state
 * update (mamba_selective_state_update) as its x (the D skip included), in
 * one kernel ("Mamba架构深度剖析：如何以线性时间重塑序列建模", §3: recurrent
 * inference, each token advancing a fixed-size state; "Mamba状态空间模型深度
 * 解析：挑战Transformer的下一代序列建模范式", §3.1: conv1d + SiLU in front of
 * the SSM).  Same result as mamba_conv1d_update followed by
 * mamba_selective_state_update, except that the conv output is not rounded to
 * `io` in between.
 *   conv_state : [B, D, K-1] of `io`, read and overwritten with the last K-1
 *                raw inputs (may be NULL when K = 1)
 *   x_raw      : [B, D] of `io`;  conv_w : [D, K] float, K in 1..4
 *                (MAMBA_MAX_FUSED_CONV_TAPS);  conv_bias : [D] float or NULL
 * Every other argument is as for mamba_selective_state_update.  y must not
 * overlap h, conv_state or any input; conv_state must not overlap h or any
 * input.
 */
mamba_status mamba_conv1d_selective_state_update(
    float *h, void *conv_state, const void *x_raw, const float *conv_w, const float *conv_bias,
    int64_t K, const void *dt, const float *dt_bias, const float *A, const void *Bm,
    const void *Cm, const float *Dskip, const void *z, void *y, int64_t B, int64_t D, int64_t N,
    mamba_dtype io, unsigned flags, void *stream);

/*
 * Backward pass of the selective scan ("Mamba状态空间模型深度解析：挑战
 * Transformer的下一代序列建模范式", §2.2: the hardware-aware algorithm
 * recomputes the intermediate states in the backward pass instead of storing
 * them).  Given the forward call's inputs and the gradient dout of its output
 * (and optionally dh_last of its final state), returns the gradients of
 *   J = sum(out * dout) + sum(h_last * dh_last)
 * with respect to every input.  Nothing from the forward call is needed
 * besides its inputs: the states are recomputed.
 *   x, dt, z, dout : [B, D, L] of `io` (z NULL: ungated forward)
 *   Bm, Cm         : [B, L, N] of `io`;  A : [D, N];  dt_bias, Dskip : [D] or NULL
 *   h0, dh_last    : [B, D, N] float or NULL (= zeros)
 *   dx, ddt        : [B, D, L] of `io`, required (ddt is the gradient of the
 *                    raw dt, before dt_bias and softplus)
 *   dz             : [B, D, L] of `io`; required when z is given, not written
 *                    when z is NULL
 *   dA             : [D, N] float, required
 *   dB, dC         : [B, L, N] float, required (summed over channels)
 *   dD, ddt_bias   : [D] float or NULL (= not returned)
 *   dh0            : [B, D, N] float or NULL (= not returned)
 *   workspace      : mamba_selective_scan_bwd_workspace_size(...) bytes,
 *                    256-byte aligned (none needed when B*D*L = 0)
 * Sums over time and channels are taken in a fixed order: the result does not
 * depend on scheduling.  Outputs must not overlap inputs, the workspace or
 * each other.  With L = 0 or B = 0 the parameter gradients are zero and dh0 =
 * dh_last.  Computed in fp32; bf16 outputs are rounded once.
 */
size_t mamba_selective_scan_bwd_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                               mamba_dtype io);

mamba_status mamba_selective_scan_bwd(
    const void *x, const void *dt, const float *dt_bias, const float *A, const void *Bm,
    const void *Cm, const float *Dskip, const void *z, const float *h0, const void *dout,
    const float *dh_last, void *dx, void *ddt, float *dA, float *dB, float *dC, float *dD,
    void *dz, float *ddt_bias, float *dh0, void *workspace, size_t workspace_bytes, int64_t B,
    int64_t D, int64_t L, int64_t N, mamba_dtype io, void *stream);

/*
 * Mamba-2 form of the scan ("SSD"): one decay value per head, shared by the
 * head's P channels and all N states, and B, C shared by a group of H/G heads.
 * The sequence map of a head is then a structured lower-triangular matrix and
 * is applied with matrix multiplications on the matrix cores
 * ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式", §4.2:
 * Mamba-2 restates the SSM as structured matrix multiplication to use the
 * GPU's matrix units).  Per (b, h, p) it computes the same recurrence as
 * mamba_selective_scan_fwd with A[d, n] = A[h] for every state n:
 *   Δ = softplus(dt[b,t,h] + dt_bias[h]),  Abar = exp(Δ A[h]),
 *   Bbar_n = (exp(Δ A[h]) - 1)/A[h] B[b,t,g,n]  (Δ B at A[h] = 0),  g = h / (H/G)
 *   h[p][n] <- Abar h[p][n] + Bbar_n x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n C[b,t,g,n] h[p][n] + Dskip[h] x[b,t,h,p]) * SiLU(z[b,t,h,p])
 *   x, z, y : [B, L, H, P] bf16 (io must be MAMBA_BF16), 16-byte aligned
 *   dt      : [B, L, H] bf16
 *   Bm, Cm  : [B, L, G, N] bf16, 16-byte aligned
 *   A       : [H] float;  dt_bias, Dskip : [H] float or NULL (= 0)
 *   z       : or NULL (= no gate)
 *   h0      : [B, H, P, N] float, 16-byte aligned, or NULL (= zeros)
 *   h_last  : [B, H, P, N] float, 16-byte aligned, or NULL (= not returned)
 * Supported: P = 64, N in {16, 32, 64, 128}, H a multiple of G; anything else
 * returns MAMBA_ERR_UNSUPPORTED (P, N, io) or MAMBA_ERR_SHAPE (G).  Needs no
 * workspace.  Products run as bf16 matrix operations with fp32 accumulation;
 * the operands that are not inputs (the scaled chunk matrix, the state, the
 * scaled x) are split into two bf16 parts, so their rounding stays near 1e-5
 * relative.  With L = 0, h_last = h0 (or zeros).
 */
mamba_status mamba_ssd_scan_fwd(const void *x, const void *dt, const float *dt_bias,
                                const float *A, const void *Bm, const void *Cm,
                                const float *Dskip, const void *z, const float *h0, void *y,
                                float *h_last, int64_t B, int64_t L, int64_t H, int64_t P,
                                int64_t G, int64_t N, mamba_dtype io, void *stream);

/*
 * Profiling hook.  When both are non-NULL hipEvent_t handles (passed as
 * void*), later calls made from this host thread record `start` right before
 * and `stop` right after the main scan kernel of mamba_selective_scan_fwd (and
 * its variants), the chunk-gradient kernel of mamba_selective_scan_bwd, or the
 * kernel of mamba_ssd_scan_fwd, on the call's stream.  Pass NULL, NULL to turn it off.
 */
void mamba_set_scan_timing_events(void *start, void *stop);

/*
 * Health of the cross-chunk carry of the calls that last used `workspace`
 * (of mamba_selective_scan_fwd and its variants, or of
 * mamba_selective_scan_bwd, whose two scans both report here).  Blocks until
 * `stream` has finished its work, then reads the workspace's error word:
 * MAMBA_OK, or MAMBA_ERR_TIMEOUT when a wait of a segment for its
 * predecessors' carry records gave up.  Such a wait is bounded (only a
 * device fault can make it time out); the segments whose start state it
 * would have given, and everything computed from them, are then NaN instead
 * of a silently wrong number.  The word is cleared by the next scan call on
 * the workspace.  MAMBA_ERR_WORKSPACE for a NULL, misaligned or too small
 * (< 256 bytes) workspace; MAMBA_ERR_LAUNCH when the stream reports an error
 * or is being captured into a graph (then nothing is waited for or read).
 */
mamba_status mamba_selective_scan_check(const void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * Diagnostic hook for tests of the failure path: polls before a carry wait of
 * later scan calls (from any host thread) gives up; polls < 0 restores the
 * default (2^22, far beyond any real wait).  With 0, any wait not satisfied at
 * its first poll gives up, so a test can make the NaN poisoning and
 * MAMBA_ERR_TIMEOUT happen while every kernel still ends normally.
 */
void mamba_set_scan_spin_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_AMD_H */
