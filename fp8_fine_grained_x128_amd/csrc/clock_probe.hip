// clock_probe.hip -- measurement support: the shader clock while other work
// runs.  One wave reads the shader-clock counter (s_memtime) and the
// constant-rate real-time counter (s_memrealtime) at the start and the end of
// a wait of `ticks` real-time ticks; launched on a second stream next to a
// running kernel, cycles / time is the clock of the CU the wave landed on.
#include <stdint.h>

#include "launch.hpp"

namespace fp8q {

// Upper bound of the wait loop (about a second of 32 x 64-cycle sleeps), so
// the wave ends even if the real-time counter were not to advance.
constexpr int kProbeMaxIters = 1 << 20;

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, uint64_t ticks,
                                                         uint64_t wall_khz) {
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r1 = r0;
    for (int i = 0; i < kProbeMaxIters && r1 - r0 < ticks; ++i) {
        __builtin_amdgcn_s_sleep(32);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[0] = r1 - r0;
        out[1] = c1 - c0;
        out[2] = wall_khz;
    }
}

hipError_t launch_clock_probe(uint64_t* out, int64_t ticks, hipStream_t st) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        khz = 0;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, st, out, (uint64_t)ticks, (uint64_t)khz);
    return hipGetLastError();
}

}  // namespace fp8q
