// VALU issue-rate probe for gfx950 (measurement aid, not part of the C ABI of
// libmamba_amd.so; built into its own libmamba_probe.so and used by
// `bench.py --probe-valu`).
//
// Each lane runs 8 independent chains for `iters` x 16 rounds, so a wave has
// enough independent instructions in flight to issue every cycle it is given.
// The occupancy (workgroups of 4 waves per CU, i.e. waves per SIMD) is set by
// the LDS each workgroup reserves, since the kernel needs few registers.
//   mode 0: v_fma_f32 on every chain (128 fp32 fmas per round per lane)
//   mode 1: v_exp_f32 then v_mul_f32 on every chain (8 + 8 per round)
//   mode 2: v_exp_f32 on chain 0, v_fma_f32 on chains 1..7 (1 + 7 per round)
// Built, like every source here, without packed fp32 instructions.
#include <hip/hip_runtime.h>

namespace {

template <int MODE, int LDS_BYTES>
__global__ void __launch_bounds__(256) valu_probe_kernel(float *out, int iters, float b, float c)
{
    __shared__ float pad[LDS_BYTES / 4];
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        a[j] = threadIdx.x * 1e-3f + j * 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (MODE == 0)
                    a[j] = fmaf(a[j], b, c);
                else if (MODE == 1)
                    a[j] = __builtin_amdgcn_exp2f(a[j]) * -0.5f;
                else
                    a[j] = (j == 0) ? __builtin_amdgcn_exp2f(a[j]) : fmaf(a[j], b, c);
            }
        }
    }
    // the LDS reservation must be used, or the compiler drops it
    pad[threadIdx.x] = a[0];
    __syncthreads();
    float s = pad[(threadIdx.x + 1) & 255];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        s += a[j];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int MODE>
hipError_t launch_mode(float *out, int grid, int wgs_per_cu, int iters, hipStream_t s)
{
    // LDS per workgroup so that exactly wgs_per_cu fit in a CU's 160 KB
    switch (wgs_per_cu) {
    case 2: hipLaunchKernelGGL((valu_probe_kernel<MODE, 75000>), dim3(grid), dim3(256), 0, s, out, iters, 0.999f, 0.001f); break;
    case 3: hipLaunchKernelGGL((valu_probe_kernel<MODE, 50000>), dim3(grid), dim3(256), 0, s, out, iters, 0.999f, 0.001f); break;
    case 4: hipLaunchKernelGGL((valu_probe_kernel<MODE, 38000>), dim3(grid), dim3(256), 0, s, out, iters, 0.999f, 0.001f); break;
    case 8: hipLaunchKernelGGL((valu_probe_kernel<MODE, 18000>), dim3(grid), dim3(256), 0, s, out, iters, 0.999f, 0.001f); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// Launches grid workgroups of 256 threads on `stream`; `out` must hold
// grid * 256 floats of device memory.  mode in {0, 1, 2}, wgs_per_cu in
// {2, 3, 4, 8}.  Returns 0, or a HIP error code (invalid mode or occupancy).
extern "C" int mamba_probe_valu_launch(float *out, int mode, int grid, int wgs_per_cu, int iters,
                                       hipStream_t stream)
{
    if (!out || grid <= 0 || iters <= 0)
        return (int)hipErrorInvalidValue;
    hipError_t e;
    switch (mode) {
    case 0: e = launch_mode<0>(out, grid, wgs_per_cu, iters, stream); break;
    case 1: e = launch_mode<1>(out, grid, wgs_per_cu, iters, stream); break;
    case 2: e = launch_mode<2>(out, grid, wgs_per_cu, iters, stream); break;
    default: e = hipErrorInvalidValue;
    }
    return (int)e;
}
