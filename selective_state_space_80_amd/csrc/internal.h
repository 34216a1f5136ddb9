// Internal declarations shared by the host API (api.cpp) and the kernel
// translation units.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mamba {

// ---- selective scan geometry -------------------------------------------------
// One wave (64 lanes) owns 64 consecutive channels of one batch row and walks a
// chunk of kChunkT time steps; kWavesPerSeg waves of a workgroup walk
// consecutive chunks, so a workgroup covers a segment of kSegT steps.
constexpr int kWave = 64;
constexpr int kChunkT = 32;
constexpr int kWavesPerSeg = 4;
constexpr int kSegT = kChunkT * kWavesPerSeg;
constexpr int kMaxN = 16;
constexpr int kAggFields = kMaxN + 1;  // decay summary + N states
constexpr int kInclFields = kMaxN;

// Byte offsets of the parts of the scan workspace for one problem shape.
struct ScanWsLayout {
    int64_t n_dtiles = 0;  // ceil(D / 64)
    int64_t groups = 0;    // B * n_dtiles
    int64_t n_seg = 0;     // ceil(L / kSegT)
    int64_t n_items = 0;   // groups * n_seg
    int64_t superseg = 0;  // segments per superblock of the carry (1: a chain)
    size_t off_header = 0, off_flags = 0, off_tiles = 0, off_agg = 0, off_incl = 0, total = 0;
};
ScanWsLayout scan_ws_layout(int64_t B, int64_t D, int64_t L);

// Classes of a 64-channel tile of A, written per call by the scan's prep kernel
// into the workspace's tile table: structured when A[d,n] = (n+1) A[d,0] with
// A[d,0] < 0 for every channel of the tile (the decays of a step are then
// powers of one exponential), general otherwise.
constexpr uint32_t kPathStructured = 0u;
constexpr uint32_t kPathGeneral = 1u;

// Byte offset of the scan workspace's error word (bit 0: a carry wait timed
// out); the header starts the workspace, also inside the backward's.
constexpr size_t kScanErrorWordOffset = 4;

// Polls (each followed by a short sleep) before a carry wait of the scan
// gives up: far beyond any real wait, so only a fault makes it happen.
constexpr int kDefaultSpinLimit = 1 << 22;

// Fused causal conv1d front end of the scan: at most this many taps.
constexpr int kFusedConvTaps = 4;

struct ScanArgs {
    const void *x, *dt, *Bm, *Cm, *z;
    const float *dt_bias, *A, *Dskip, *h0;
    void *y;
    float *h_last;
    unsigned char *ws;
    ScanWsLayout lay;
    int64_t B, D, L;
    int N;
    bool bf16;
    // fused front end (conv_K = 0: x is the scan input itself; else x is the
    // raw input and the scan input is SiLU(causal conv1d(x)))
    int conv_K;
    const float *conv_w, *conv_b;
    const void *conv_state_in;
    void *conv_state_out;
    bool reverse;     // scan from step L-1 down to step 0 (plain scan only)
    bool accumulate;  // y += result
    // backward pass helpers: adjoint = the reverse scan of the adjoint state
    // nu_t = Abar_t (nu_(t+1) + C_t dy_t) with x = dout (y unused; h0 = the
    // final state's gradient, h_last = dh0); chunk_states = per 32-step chunk
    // its start state in scan order, [groups][n_seg*4][16][64] floats
    bool adjoint = false;
    float *chunk_states = nullptr;
    // the workspace's error word keeps an earlier scan's timeout (the second
    // scan of a backward call) instead of starting from zero
    bool keep_error = false;
    int spin_limit = kDefaultSpinLimit;  // polls before a carry wait gives up
    hipEvent_t ev_start, ev_stop;  // optional timing of the main kernel
};
hipError_t launch_selective_scan(const ScanArgs &a, hipStream_t s);

// Backward pass of the scan (scan_bwd.hip).  Gradients of sum(out * dout)
// (+ sum(h_last * dh_last)); see launch_selective_scan_bwd.
struct BwdWsLayout {
    ScanWsLayout scan;  // the two scans' workspace (forward, then adjoint)
    size_t off_hsave = 0, off_nusave = 0, off_dBp = 0, off_dCp = 0, off_dAp = 0, off_dDp = 0,
           off_dbp = 0, total = 0;
};
BwdWsLayout scan_bwd_ws_layout(int64_t B, int64_t D, int64_t L);

struct BwdArgsHost {
    const void *x, *dt, *Bm, *Cm, *z, *dout;
    const float *dt_bias, *A, *Dskip, *h0, *dh_last;
    void *dx, *ddt, *dz;                          // [B, D, L] of the I/O type
    float *dA, *dB, *dC, *dD, *ddt_bias, *dh0;    // fp32
    unsigned char *ws;
    int64_t B, D, L;
    int N;
    bool bf16;
    hipEvent_t ev_start, ev_stop;  // optional timing of the chunk-gradient kernel
    int spin_limit = kDefaultSpinLimit;  // of the two scans' carry waits
};
hipError_t launch_selective_scan_bwd(const BwdArgsHost &a, hipStream_t s);

// Mamba-2 form (ssd_fwd.hip): one decay per head, B/C per group of heads.
constexpr int kSsdHeadDim = 64;  // channels per head (P)
struct SsdArgs {
    const void *x, *dt, *Bm, *Cm, *z;  // bf16: x, z, y [B, L, H, P]; dt [B, L, H]; B, C [B, L, G, N]
    const float *dt_bias, *A, *Dskip, *h0;  // [H], [H], [H], [B, H, P, N]
    void *y;
    float *h_last;  // [B, H, P, N] or NULL
    int64_t B, L, H, G;
    int N;
    hipEvent_t ev_start, ev_stop;  // optional timing of the kernel
};
hipError_t launch_ssd_fwd(const SsdArgs &a, hipStream_t s);

struct ConvArgs {
    const void *x;
    const float *w, *bias;
    void *out;
    int64_t B, D, L;
    int K;
    bool bf16;
};
hipError_t launch_conv1d_silu(const ConvArgs &a, hipStream_t s);

struct ConvUpdateArgs {
    void *state;  // [B, D, K-1] of the I/O type, in/out
    const void *x;
    const float *w, *bias;
    void *out;
    int64_t B, D;
    int K;
    bool bf16;
};
hipError_t launch_conv1d_update(const ConvUpdateArgs &a, hipStream_t s);

struct StepArgs {
    float *h;
    const void *x, *dt, *Bm, *Cm, *z;
    const float *dt_bias, *A, *Dskip;
    void *y;
    int64_t B, D;
    int N;
    bool bf16;
    // conv front end in front (conv_K in 1..kFusedConvTaps; 0 = none): x is
    // the raw input and conv_state [B, D, K-1] its window, updated in place
    int conv_K = 0;
    void *conv_state = nullptr;
    const float *conv_w = nullptr, *conv_b = nullptr;
    // h loaded and stored with nontemporal hints (MAMBA_STEP_STREAM_STATE)
    bool stream_state = false;
};
hipError_t launch_state_update(const StepArgs &a, hipStream_t s);

}  // namespace mamba
