// Host side of the C ABI declared in include/mamba_amd.h: argument
// validation (before any HIP call), workspace sizing, and launch.
#include "mamba_amd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <atomic>
#include <mutex>

#include "internal.h"

namespace {

using mamba::kMaxN;

constexpr int64_t kMaxElems = int64_t(1) << 40;  // B*D*L bound (keeps every index in int64)
// Every launch keeps blocks x threads per grid dimension below 2^32 work-items;
// the MAMBA_ERR_SHAPE checks below bound each entry point's grids for that.
constexpr int64_t kMaxGrid = int64_t(1) << 31;

thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;
std::atomic<int> g_spin_limit{mamba::kDefaultSpinLimit};

bool valid_dtype(int dt) { return dt == MAMBA_F32 || dt == MAMBA_BF16; }
size_t esize(mamba_dtype dt) { return dt == MAMBA_BF16 ? 2 : 4; }

bool aligned(const void *p, size_t a) { return p == nullptr || (uintptr_t)p % a == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range rng(const void *p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b)
{
    if (a.lo == 0 || b.lo == 0 || a.hi == a.lo || b.hi == b.lo)
        return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// Non-negative sizes; each, and the product of the non-zero ones, at most
// kMaxElems (so an empty dimension leaves the others bounded too).
bool sizes_ok(int64_t a, int64_t b, int64_t c)
{
    if (a < 0 || b < 0 || c < 0)
        return false;
    int64_t p = 1;
    for (const int64_t v : {a, b, c}) {
        if (v == 0)
            continue;
        if (v > kMaxElems || p > kMaxElems / v)
            return false;
        p *= v;
    }
    return true;
}

// The kernels are built for gfx950 only.
mamba_status device_ok()
{
    static std::mutex mu;
    static int checked[64] = {0};  // 0 unknown, 1 ok, 2 bad
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return MAMBA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 64)
        return MAMBA_ERR_DEVICE;
    if (checked[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return MAMBA_ERR_DEVICE;
        checked[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    return checked[dev] == 1 ? MAMBA_OK : MAMBA_ERR_DEVICE;
}

mamba_status launched(hipError_t e) { return e == hipSuccess ? MAMBA_OK : MAMBA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *mamba_status_string(int status)
{
    switch (status) {
    case MAMBA_OK: return "MAMBA_OK";
    case MAMBA_ERR_NULL: return "MAMBA_ERR_NULL: a required pointer is NULL";
    case MAMBA_ERR_SHAPE: return "MAMBA_ERR_SHAPE: negative size or problem too large";
    case MAMBA_ERR_DTYPE: return "MAMBA_ERR_DTYPE: dtype must be MAMBA_F32 or MAMBA_BF16";
    case MAMBA_ERR_UNSUPPORTED:
        return "MAMBA_ERR_UNSUPPORTED: a size, type or flag this entry point does not take "
               "(scan: N 1..16; conv: K 1..8, 1..4 fused; Mamba-2 form: bf16, P 64, "
               "N 16/32/64/128)";
    case MAMBA_ERR_ALIGN: return "MAMBA_ERR_ALIGN: pointer not aligned to its element size";
    case MAMBA_ERR_ALIAS: return "MAMBA_ERR_ALIAS: an output overlaps an input";
    case MAMBA_ERR_WORKSPACE: return "MAMBA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MAMBA_ERR_LAUNCH: return "MAMBA_ERR_LAUNCH: HIP failed to launch a kernel";
    case MAMBA_ERR_DEVICE: return "MAMBA_ERR_DEVICE: no gfx950 HIP device is current";
    case MAMBA_ERR_TIMEOUT: return "MAMBA_ERR_TIMEOUT: a carry wait of the scan gave up (outputs poisoned with NaN)";
    default: return "unknown mamba_status";
    }
}

int mamba_abi_version(void) { return MAMBA_AMD_ABI_VERSION; }

void mamba_set_scan_spin_limit(int polls)
{
    g_spin_limit.store(polls < 0 ? mamba::kDefaultSpinLimit : polls);
}

mamba_status mamba_selective_scan_check(const void *workspace, size_t workspace_bytes,
                                        void *stream)
{
    if (!workspace || workspace_bytes < 256 || !aligned(workspace, 256))
        return MAMBA_ERR_WORKSPACE;
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &cap) != hipSuccess ||
        cap != hipStreamCaptureStatusNone)
        return MAMBA_ERR_LAUNCH;  // a stream under graph capture cannot be waited for
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return MAMBA_ERR_LAUNCH;
    uint32_t word = 0;
    if (hipMemcpy(&word, (const unsigned char *)workspace + mamba::kScanErrorWordOffset,
                  sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return MAMBA_ERR_LAUNCH;
    return word ? MAMBA_ERR_TIMEOUT : MAMBA_OK;
}

void mamba_set_scan_timing_events(void *start, void *stop)
{
    if (start && stop) {
        g_ev_start = (hipEvent_t)start;
        g_ev_stop = (hipEvent_t)stop;
    } else {
        g_ev_start = nullptr;
        g_ev_stop = nullptr;
    }
}

mamba_status mamba_conv1d_silu(const void *x, const float *w, const float *bias, void *out,
                               int64_t B, int64_t D, int64_t L, int64_t K, mamba_dtype dtype,
                               void *stream)
{
    if (!valid_dtype(dtype))
        return MAMBA_ERR_DTYPE;
    if (!sizes_ok(B, D, L) || K < 0)
        return MAMBA_ERR_SHAPE;
    if (K < 1 || K > MAMBA_MAX_CONV_TAPS)
        return MAMBA_ERR_UNSUPPORTED;
    if (B * D * ((L + 3) / 4) >= kMaxGrid)  // launch grid: one thread per 4 or 8 steps
        return MAMBA_ERR_SHAPE;
    const int64_t n = B * D * L;
    if (n == 0)
        return MAMBA_OK;
    if (!x || !w || !out)
        return MAMBA_ERR_NULL;
    const size_t es = esize(dtype);
    if (!aligned(x, es) || !aligned(out, es) || !aligned(w, 4) || !aligned(bias, 4))
        return MAMBA_ERR_ALIGN;
    const Range ro = rng(out, (size_t)n * es);
    if (overlap(ro, rng(x, (size_t)n * es)) || overlap(ro, rng(w, (size_t)(D * K) * 4)) ||
        (bias && overlap(ro, rng(bias, (size_t)D * 4))))
        return MAMBA_ERR_ALIAS;
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    mamba::ConvArgs a{x, w, bias, out, B, D, L, (int)K, dtype == MAMBA_BF16};
    return launched(mamba::launch_conv1d_silu(a, (hipStream_t)stream));
}

size_t mamba_selective_scan_fwd_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                               mamba_dtype io)
{
    (void)io;
    if (!sizes_ok(B, D, L) || N < 1 || N > kMaxN)
        return 0;
    if (B * D * L == 0)
        return 0;
    return mamba::scan_ws_layout(B, D, L).total;
}

}  // extern "C"

namespace {

// Shared body of the two scan entry points.  conv_K = 0: x is the scan input;
// conv_K in 1..4: x is the raw input of the fused conv1d + SiLU front end.
mamba_status scan_entry(const void *x, int64_t conv_K, const float *conv_w,
                        const float *conv_b, const void *conv_state_in, void *conv_state_out,
                        const void *dt, const float *dt_bias, const float *A, const void *Bm,
                        const void *Cm, const float *Dskip, const void *z, const float *h0,
                        void *y, float *h_last, void *workspace, size_t workspace_bytes,
                        int64_t B, int64_t D, int64_t L, int64_t N, mamba_dtype io,
                        unsigned flags, void *stream)
{
    if (!valid_dtype(io))
        return MAMBA_ERR_DTYPE;
    if (!sizes_ok(B, D, L) || N < 0 || conv_K < 0)
        return MAMBA_ERR_SHAPE;
    if (N < 1 || N > kMaxN)
        return MAMBA_ERR_UNSUPPORTED;
    const bool conv = conv_K != 0;
    if ((flags & ~(unsigned)(MAMBA_SCAN_REVERSE | MAMBA_SCAN_ACCUMULATE)) != 0 ||
        (conv && (flags & MAMBA_SCAN_REVERSE)))
        return MAMBA_ERR_UNSUPPORTED;
    if (conv && conv_K > mamba::kFusedConvTaps)
        return MAMBA_ERR_UNSUPPORTED;
    if (L == 0 && (h_last || conv_state_out) && B * D * N >= kMaxGrid)
        return MAMBA_ERR_SHAPE;  // launch grid of the state copy
    if (B * D == 0)
        return MAMBA_OK;
    const int64_t n = B * D * L;
    const size_t es = esize(io);
    const size_t cs_bytes = conv ? (size_t)(B * D * (conv_K - 1)) * es : 0;
    const Range r_csin = rng(conv_state_in, conv_state_in ? cs_bytes : 0);
    const Range r_csout = rng(conv_state_out, conv_state_out ? cs_bytes : 0);
    if (conv) {
        if (!conv_w)
            return MAMBA_ERR_NULL;
        if (!aligned(conv_w, 4) || !aligned(conv_b, 4) || !aligned(conv_state_in, es) ||
            !aligned(conv_state_out, es))
            return MAMBA_ERR_ALIGN;
    }
    if (L == 0) {
        // nothing to scan; h_last (if asked for) is the initial state, the
        // conv state (if asked for) the carried-in one
        if (!aligned(h_last, 4) || !aligned(h0, 4))
            return MAMBA_ERR_ALIGN;
        const Range rh = rng(h_last, h_last ? (size_t)(B * D * N) * 4 : 0);
        if (h0 && overlap(rh, rng(h0, (size_t)(B * D * N) * 4)))
            return MAMBA_ERR_ALIAS;
        if (overlap(r_csout, rh) || overlap(r_csout, rng(h0, h0 ? (size_t)(B * D * N) * 4 : 0)) ||
            overlap(r_csin, rh))
            return MAMBA_ERR_ALIAS;
        if (!h_last && !conv_state_out)
            return MAMBA_OK;
    } else {
        if (!x || !dt || !A || !Bm || !Cm || !y)
            return MAMBA_ERR_NULL;
        if (!aligned(x, es) || !aligned(dt, es) || !aligned(z, es) || !aligned(y, es) ||
            !aligned(Bm, es) || !aligned(Cm, es) || !aligned(A, 4) || !aligned(dt_bias, 4) ||
            !aligned(Dskip, 4) || !aligned(h0, 4) || !aligned(h_last, 4))
            return MAMBA_ERR_ALIGN;
        if (B * L * kMaxN >= (int64_t(1) << 31))
            return MAMBA_ERR_SHAPE;
        const mamba::ScanWsLayout lay = mamba::scan_ws_layout(B, D, L);
        if (lay.n_items >= (int64_t(1) << 23))
            return MAMBA_ERR_SHAPE;
        if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256))
            return MAMBA_ERR_WORKSPACE;
        const Range ry = rng(y, (size_t)n * es);
        const Range rh = rng(h_last, h_last ? (size_t)(B * D * N) * 4 : 0);
        const Range rw = rng(workspace, lay.total);
        const Range ins[] = {rng(x, (size_t)n * es),          rng(dt, (size_t)n * es),
                             rng(z, z ? (size_t)n * es : 0),  rng(Bm, (size_t)(B * L * N) * es),
                             rng(Cm, (size_t)(B * L * N) * es), rng(A, (size_t)(D * N) * 4),
                             rng(dt_bias, dt_bias ? (size_t)D * 4 : 0),
                             rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                             rng(h0, h0 ? (size_t)(B * D * N) * 4 : 0),
                             rng(conv_w, conv ? (size_t)(D * conv_K) * 4 : 0),
                             rng(conv_b, conv && conv_b ? (size_t)D * 4 : 0),
                             r_csin};
        for (const Range &r : ins)
            if (overlap(ry, r) || overlap(rh, r) || overlap(rw, r))
                return MAMBA_ERR_ALIAS;
        if (overlap(ry, rh) || overlap(ry, rw) || overlap(rh, rw))
            return MAMBA_ERR_ALIAS;
        // the conv state out may only share memory with the conv state in
        for (const Range &r : ins)
            if (!(r.lo == r_csin.lo && r.hi == r_csin.hi) && overlap(r_csout, r))
                return MAMBA_ERR_ALIAS;
        if (overlap(r_csout, ry) || overlap(r_csout, rh) || overlap(r_csout, rw))
            return MAMBA_ERR_ALIAS;
    }
    // a conv state out that overlaps the one in must be the very same buffer
    if (overlap(r_csout, r_csin) && !(r_csout.lo == r_csin.lo && r_csout.hi == r_csin.hi))
        return MAMBA_ERR_ALIAS;
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    mamba::ScanArgs a;
    a.x = x;
    a.dt = dt;
    a.Bm = Bm;
    a.Cm = Cm;
    a.z = z;
    a.dt_bias = dt_bias;
    a.A = A;
    a.Dskip = Dskip;
    a.h0 = h0;
    a.y = y;
    a.h_last = h_last;
    a.ws = (unsigned char *)workspace;
    a.lay = mamba::scan_ws_layout(B, D, L);
    a.B = B;
    a.D = D;
    a.L = L;
    a.N = (int)N;
    a.bf16 = io == MAMBA_BF16;
    a.conv_K = (int)conv_K;
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.conv_state_in = conv_state_in;
    a.conv_state_out = conv_state_out;
    a.reverse = (flags & MAMBA_SCAN_REVERSE) != 0;
    a.accumulate = (flags & MAMBA_SCAN_ACCUMULATE) != 0;
    a.ev_start = g_ev_start;
    a.ev_stop = g_ev_stop;
    a.spin_limit = g_spin_limit.load();
    return launched(mamba::launch_selective_scan(a, (hipStream_t)stream));
}

// Shared body of the two decode entry points.  conv_K = 0: x is the scan
// input; conv_K in 1..4: x is the raw input of the fused conv front end, whose
// window conv_state is updated in place.
mamba_status step_entry(float *h, void *conv_state, const void *x, int64_t conv_K,
                        const float *conv_w, const float *conv_b, const void *dt,
                        const float *dt_bias, const float *A, const void *Bm, const void *Cm,
                        const float *Dskip, const void *z, void *y, int64_t B, int64_t D,
                        int64_t N, mamba_dtype io, unsigned flags, void *stream)
{
    if (!valid_dtype(io))
        return MAMBA_ERR_DTYPE;
    if (!sizes_ok(B, D, 1) || N < 0 || conv_K < 0)
        return MAMBA_ERR_SHAPE;
    if (N < 1 || N > kMaxN || conv_K > mamba::kFusedConvTaps)
        return MAMBA_ERR_UNSUPPORTED;
    if ((flags & ~(unsigned)MAMBA_STEP_STREAM_STATE) != 0)
        return MAMBA_ERR_UNSUPPORTED;
    if (B * D >= kMaxGrid)  // launch grid: up to two lanes per channel in a row's dimension
        return MAMBA_ERR_SHAPE;
    if (B * D == 0)
        return MAMBA_OK;
    const bool conv = conv_K != 0;
    if (!h || !x || !dt || !A || !Bm || !Cm || !y || (conv && !conv_w) ||
        (conv_K > 1 && !conv_state))
        return MAMBA_ERR_NULL;
    const size_t es = esize(io);
    if (!aligned(h, 4) || !aligned(x, es) || !aligned(dt, es) || !aligned(z, es) ||
        !aligned(y, es) || !aligned(Bm, es) || !aligned(Cm, es) || !aligned(A, 4) ||
        !aligned(dt_bias, 4) || !aligned(Dskip, 4) || !aligned(conv_state, es) ||
        !aligned(conv_w, 4) || !aligned(conv_b, 4))
        return MAMBA_ERR_ALIGN;
    const int64_t n = B * D;
    const Range ry = rng(y, (size_t)n * es);
    const Range rh = rng(h, (size_t)(n * N) * 4);
    const Range rc = rng(conv_state, conv_K > 1 ? (size_t)(n * (conv_K - 1)) * es : 0);
    const Range ins[] = {rng(x, (size_t)n * es), rng(dt, (size_t)n * es),
                         rng(z, z ? (size_t)n * es : 0), rng(Bm, (size_t)(B * N) * es),
                         rng(Cm, (size_t)(B * N) * es), rng(A, (size_t)(D * N) * 4),
                         rng(dt_bias, dt_bias ? (size_t)D * 4 : 0),
                         rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                         rng(conv_w, conv ? (size_t)(D * conv_K) * 4 : 0),
                         rng(conv_b, conv && conv_b ? (size_t)D * 4 : 0)};
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rh, r) || overlap(rc, r))
            return MAMBA_ERR_ALIAS;
    if (overlap(ry, rh) || overlap(ry, rc) || overlap(rh, rc))
        return MAMBA_ERR_ALIAS;
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    mamba::StepArgs a{h, x, dt, Bm, Cm, z, dt_bias, A, Dskip, y, B, D, (int)N, io == MAMBA_BF16};
    a.conv_K = (int)conv_K;
    a.conv_state = conv_state;
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.stream_state = (flags & MAMBA_STEP_STREAM_STATE) != 0;
    return launched(mamba::launch_state_update(a, (hipStream_t)stream));
}

// ---- scratch of the entry point that allocates nothing ----------------------
// The workspace of mamba_selective_scan_fwd_noalloc: a file-scope device array
// that every GPU the library runs on holds until the process ends.  In host
// code its name is only a stand-in, not a device address: the address of each
// device's copy comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MAMBA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {nullptr};

// This device's copy of `scratch` (NULL if its address cannot be had).
void *scratch_of_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

mamba_status mamba_selective_scan_fwd_noalloc(const void *x, const void *dt,
                                              const float *dt_bias, const float *A,
                                              const void *Bm, const void *Cm,
                                              const float *Dskip, const void *z,
                                              const float *h0, void *y, float *h_last,
                                              int64_t B, int64_t D, int64_t L, int64_t N,
                                              mamba_dtype io, void *stream)
{
    // the shape's workspace must fit the scratch (0 = nothing to scan)
    if (sizes_ok(B, D, L) && N >= 1 && N <= kMaxN && B * D * L > 0 &&
        mamba::scan_ws_layout(B, D, L).total > (size_t)MAMBA_NOALLOC_SCRATCH_BYTES)
        return MAMBA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (sizes_ok(B, D, L) && B * D * L > 0) {
        const mamba_status st = device_ok();
        if (st != MAMBA_OK)
            return st;
        ws = scratch_of_current_device();
        if (!ws)
            return MAMBA_ERR_DEVICE;
    }
    return scan_entry(x, 0, nullptr, nullptr, nullptr, nullptr, dt, dt_bias, A, Bm, Cm, Dskip,
                      z, h0, y, h_last, ws, ws ? (size_t)MAMBA_NOALLOC_SCRATCH_BYTES : 0, B, D,
                      L, N, io, 0u, stream);
}

mamba_status mamba_selective_scan_fwd(const void *x, const void *dt, const float *dt_bias,
                                      const float *A, const void *Bm, const void *Cm,
                                      const float *Dskip, const void *z, const float *h0,
                                      void *y, float *h_last, void *workspace,
                                      size_t workspace_bytes, int64_t B, int64_t D, int64_t L,
                                      int64_t N, mamba_dtype io, void *stream)
{
    return scan_entry(x, 0, nullptr, nullptr, nullptr, nullptr, dt, dt_bias, A, Bm, Cm, Dskip,
                      z, h0, y, h_last, workspace, workspace_bytes, B, D, L, N, io, 0u, stream);
}

mamba_status mamba_selective_scan_fwd_ex(const void *x, const void *dt, const float *dt_bias,
                                         const float *A, const void *Bm, const void *Cm,
                                         const float *Dskip, const void *z, const float *h0,
                                         void *y, float *h_last, void *workspace,
                                         size_t workspace_bytes, int64_t B, int64_t D, int64_t L,
                                         int64_t N, mamba_dtype io, unsigned flags, void *stream)
{
    return scan_entry(x, 0, nullptr, nullptr, nullptr, nullptr, dt, dt_bias, A, Bm, Cm, Dskip,
                      z, h0, y, h_last, workspace, workspace_bytes, B, D, L, N, io, flags,
                      stream);
}

mamba_status mamba_conv1d_selective_scan_fwd(
    const void *x_raw, const float *conv_w, const float *conv_bias, int64_t K,
    const void *conv_state_in, void *conv_state_out, const void *dt, const float *dt_bias,
    const float *A, const void *Bm, const void *Cm, const float *Dskip, const void *z,
    const float *h0, void *y, float *h_last, void *workspace, size_t workspace_bytes, int64_t B,
    int64_t D, int64_t L, int64_t N, mamba_dtype io, void *stream)
{
    if (K < 0)
        return valid_dtype(io) ? MAMBA_ERR_SHAPE : MAMBA_ERR_DTYPE;
    if (K == 0)
        return valid_dtype(io) ? MAMBA_ERR_UNSUPPORTED : MAMBA_ERR_DTYPE;
    return scan_entry(x_raw, K, conv_w, conv_bias, conv_state_in, conv_state_out, dt, dt_bias, A,
                      Bm, Cm, Dskip, z, h0, y, h_last, workspace, workspace_bytes, B, D, L, N, io,
                      0u, stream);
}

mamba_status mamba_conv1d_update(void *state, const void *x, const float *w, const float *bias,
                                 void *out, int64_t B, int64_t D, int64_t K, mamba_dtype dtype,
                                 void *stream)
{
    if (!valid_dtype(dtype))
        return MAMBA_ERR_DTYPE;
    if (!sizes_ok(B, D, 1) || K < 0)
        return MAMBA_ERR_SHAPE;
    if (K < 1 || K > MAMBA_MAX_CONV_TAPS)
        return MAMBA_ERR_UNSUPPORTED;
    if (B * D >= kMaxGrid)  // launch grid: up to one thread per channel
        return MAMBA_ERR_SHAPE;
    const int64_t n = B * D;
    if (n == 0)
        return MAMBA_OK;
    if (!x || !w || !out || (K > 1 && !state))
        return MAMBA_ERR_NULL;
    const size_t es = esize(dtype);
    if (!aligned(state, es) || !aligned(x, es) || !aligned(out, es) || !aligned(w, 4) ||
        !aligned(bias, 4))
        return MAMBA_ERR_ALIGN;
    const Range ro = rng(out, (size_t)n * es);
    const Range rs = rng(state, K > 1 ? (size_t)(n * (K - 1)) * es : 0);
    const Range ins[] = {rng(x, (size_t)n * es), rng(w, (size_t)(D * K) * 4),
                         rng(bias, bias ? (size_t)D * 4 : 0)};
    for (const Range &r : ins)
        if (overlap(ro, r) || overlap(rs, r))
            return MAMBA_ERR_ALIAS;
    if (overlap(ro, rs))
        return MAMBA_ERR_ALIAS;
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    mamba::ConvUpdateArgs a{state, x, w, bias, out, B, D, (int)K, dtype == MAMBA_BF16};
    return launched(mamba::launch_conv1d_update(a, (hipStream_t)stream));
}

mamba_status mamba_selective_state_update(float *h, const void *x, const void *dt,
                                          const float *dt_bias, const float *A,
                                          const void *Bm, const void *Cm, const float *Dskip,
                                          const void *z, void *y, int64_t B, int64_t D,
                                          int64_t N, mamba_dtype io, unsigned flags,
                                          void *stream)
{
    return step_entry(h, nullptr, x, 0, nullptr, nullptr, dt, dt_bias, A, Bm, Cm, Dskip, z, y, B,
                      D, N, io, flags, stream);
}

mamba_status mamba_conv1d_selective_state_update(
    float *h, void *conv_state, const void *x_raw, const float *conv_w, const float *conv_bias,
    int64_t K, const void *dt, const float *dt_bias, const float *A, const void *Bm,
    const void *Cm, const float *Dskip, const void *z, void *y, int64_t B, int64_t D, int64_t N,
    mamba_dtype io, unsigned flags, void *stream)
{
    if (K < 0)
        return valid_dtype(io) ? MAMBA_ERR_SHAPE : MAMBA_ERR_DTYPE;
    if (K == 0)
        return valid_dtype(io) ? MAMBA_ERR_UNSUPPORTED : MAMBA_ERR_DTYPE;
    return step_entry(h, conv_state, x_raw, K, conv_w, conv_bias, dt, dt_bias, A, Bm, Cm, Dskip,
                      z, y, B, D, N, io, flags, stream);
}

size_t mamba_selective_scan_bwd_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                               mamba_dtype io)
{
    (void)io;
    if (!sizes_ok(B, D, L) || N < 1 || N > kMaxN)
        return 0;
    if (B * D * L == 0)
        return 0;
    return mamba::scan_bwd_ws_layout(B, D, L).total;
}

mamba_status mamba_selective_scan_bwd(
    const void *x, const void *dt, const float *dt_bias, const float *A, const void *Bm,
    const void *Cm, const float *Dskip, const void *z, const float *h0, const void *dout,
    const float *dh_last, void *dx, void *ddt, float *dA, float *dB, float *dC, float *dD,
    void *dz, float *ddt_bias, float *dh0, void *workspace, size_t workspace_bytes, int64_t B,
    int64_t D, int64_t L, int64_t N, mamba_dtype io, void *stream)
{
    if (!valid_dtype(io))
        return MAMBA_ERR_DTYPE;
    if (!sizes_ok(B, D, L) || N < 0)
        return MAMBA_ERR_SHAPE;
    if (N < 1 || N > kMaxN)
        return MAMBA_ERR_UNSUPPORTED;
    if (D == 0)
        return MAMBA_OK;
    const bool empty = B * L == 0;
    if (!dA)
        return MAMBA_ERR_NULL;
    if (!empty && (!x || !dt || !A || !Bm || !Cm || !dout || !dx || !ddt || !dB || !dC ||
                   (z && !dz)))
        return MAMBA_ERR_NULL;
    if (!z)
        dz = nullptr;  // no gate, no gate gradient
    const size_t es = esize(io);
    if (!aligned(x, es) || !aligned(dt, es) || !aligned(z, es) || !aligned(dout, es) ||
        !aligned(Bm, es) || !aligned(Cm, es) || !aligned(dx, es) || !aligned(ddt, es) ||
        !aligned(dz, es) || !aligned(A, 4) || !aligned(dt_bias, 4) || !aligned(Dskip, 4) ||
        !aligned(h0, 4) || !aligned(dh_last, 4) || !aligned(dA, 4) || !aligned(dB, 4) ||
        !aligned(dC, 4) || !aligned(dD, 4) || !aligned(ddt_bias, 4) || !aligned(dh0, 4))
        return MAMBA_ERR_ALIGN;
    if (empty && (B * D * N >= kMaxGrid || D * N >= kMaxGrid))  // grid of the empty-problem kernel
        return MAMBA_ERR_SHAPE;
    size_t ws_need = 0;
    if (!empty) {
        if (B * L * kMaxN >= (int64_t(1) << 31))
            return MAMBA_ERR_SHAPE;
        const mamba::BwdWsLayout lay = mamba::scan_bwd_ws_layout(B, D, L);
        // chunk kernel: four 32-step chunks per segment, 256 threads each;
        // column sums: up to 16 threads per (b, t, n) column
        if (lay.scan.n_items >= (int64_t(1) << 21) || B * L >= (int64_t(1) << 25))
            return MAMBA_ERR_SHAPE;
        ws_need = lay.total;
        if (!workspace || workspace_bytes < ws_need || !aligned(workspace, 256))
            return MAMBA_ERR_WORKSPACE;
    }
    const int64_t n = B * D * L;
    const size_t nb = (size_t)n * es, bln = (size_t)(B * L * N) * 4, dn = (size_t)(D * N) * 4,
                 bdn = (size_t)(B * D * N) * 4;
    const Range ins[] = {rng(x, x ? nb : 0),
                         rng(dt, dt ? nb : 0),
                         rng(z, z ? nb : 0),
                         rng(dout, dout ? nb : 0),
                         rng(Bm, Bm ? (size_t)(B * L * N) * es : 0),
                         rng(Cm, Cm ? (size_t)(B * L * N) * es : 0),
                         rng(A, A ? dn : 0),
                         rng(dt_bias, dt_bias ? (size_t)D * 4 : 0),
                         rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                         rng(h0, h0 ? bdn : 0),
                         rng(dh_last, dh_last ? bdn : 0)};
    const Range outs[] = {rng(dx, dx ? nb : 0),
                          rng(ddt, ddt ? nb : 0),
                          rng(dz, dz ? nb : 0),
                          rng(dA, dn),
                          rng(dB, dB ? bln : 0),
                          rng(dC, dC ? bln : 0),
                          rng(dD, dD ? (size_t)D * 4 : 0),
                          rng(ddt_bias, ddt_bias ? (size_t)D * 4 : 0),
                          rng(dh0, dh0 ? bdn : 0),
                          rng(workspace, ws_need)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r))
                return MAMBA_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j]))
                return MAMBA_ERR_ALIAS;
    }
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    mamba::BwdArgsHost a;
    a.x = x;
    a.dt = dt;
    a.Bm = Bm;
    a.Cm = Cm;
    a.z = z;
    a.dout = dout;
    a.dt_bias = dt_bias;
    a.A = A;
    a.Dskip = Dskip;
    a.h0 = h0;
    a.dh_last = dh_last;
    a.dx = dx;
    a.ddt = ddt;
    a.dz = dz;
    a.dA = dA;
    a.dB = dB;
    a.dC = dC;
    a.dD = dD;
    a.ddt_bias = ddt_bias;
    a.dh0 = dh0;
    a.ws = (unsigned char *)workspace;
    a.B = B;
    a.D = D;
    a.L = L;
    a.N = (int)N;
    a.bf16 = io == MAMBA_BF16;
    a.ev_start = g_ev_start;
    a.ev_stop = g_ev_stop;
    a.spin_limit = g_spin_limit.load();
    return launched(mamba::launch_selective_scan_bwd(a, (hipStream_t)stream));
}

mamba_status mamba_ssd_scan_fwd(const void *x, const void *dt, const float *dt_bias,
                                const float *A, const void *Bm, const void *Cm,
                                const float *Dskip, const void *z, const float *h0, void *y,
                                float *h_last, int64_t B, int64_t L, int64_t H, int64_t P,
                                int64_t G, int64_t N, mamba_dtype io, void *stream)
{
    if (!valid_dtype(io))
        return MAMBA_ERR_DTYPE;
    if (!sizes_ok(B, L, H) || P < 0 || N < 0 || G < 0 || !sizes_ok(B * L, H, P))
        return MAMBA_ERR_SHAPE;
    if (io != MAMBA_BF16 || P != mamba::kSsdHeadDim || !(N == 16 || N == 32 || N == 64 || N == 128))
        return MAMBA_ERR_UNSUPPORTED;
    if (G < 1 || H % G != 0 || B * H >= (int64_t(1) << 24))  // one 256-thread workgroup each
        return MAMBA_ERR_SHAPE;
    if (H * P * 64 >= (int64_t(1) << 31) || G * N * 64 >= (int64_t(1) << 31))
        return MAMBA_ERR_SHAPE;  // 32-bit offsets within a 64-step chunk
    if (B * H == 0)
        return MAMBA_OK;
    if (!A || (L > 0 && (!x || !dt || !Bm || !Cm || !y)))
        return MAMBA_ERR_NULL;
    if (L == 0 && !h_last)
        return MAMBA_OK;
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(Bm, 16) ||
        !aligned(Cm, 16) || !aligned(dt, 2) || !aligned(A, 4) || !aligned(dt_bias, 4) ||
        !aligned(Dskip, 4) || !aligned(h0, 16) || !aligned(h_last, 16))
        return MAMBA_ERR_ALIGN;
    const size_t nx = (size_t)(B * L * H * P) * 2, nbc = (size_t)(B * L * G * N) * 2,
                 ns = (size_t)(B * H * P * N) * 4;
    const Range ry = rng(y, L > 0 ? nx : 0), rh = rng(h_last, h_last ? ns : 0);
    const Range ins[] = {rng(x, L > 0 ? nx : 0), rng(dt, (size_t)(B * L * H) * 2),
                         rng(z, z && L > 0 ? nx : 0), rng(Bm, nbc), rng(Cm, nbc),
                         rng(A, (size_t)H * 4), rng(dt_bias, dt_bias ? (size_t)H * 4 : 0),
                         rng(Dskip, Dskip ? (size_t)H * 4 : 0), rng(h0, h0 ? ns : 0)};
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rh, r))
            return MAMBA_ERR_ALIAS;
    if (overlap(ry, rh))
        return MAMBA_ERR_ALIAS;
    mamba_status st = device_ok();
    if (st != MAMBA_OK)
        return st;
    mamba::SsdArgs a;
    a.x = x;
    a.dt = dt;
    a.Bm = Bm;
    a.Cm = Cm;
    a.z = z;
    a.dt_bias = dt_bias;
    a.A = A;
    a.Dskip = Dskip;
    a.h0 = h0;
    a.y = y;
    a.h_last = h_last;
    a.B = B;
    a.L = L;
    a.H = H;
    a.G = G;
    a.N = (int)N;
    a.ev_start = g_ev_start;
    a.ev_stop = g_ev_stop;
    return launched(mamba::launch_ssd_fwd(a, (hipStream_t)stream));
}

}  // extern "C"
