// validate_driver.cpp -- runs the C ABI's host-side argument checks
// (validate.hpp) on fixed cases with known answers and on a large seeded
// sample of argument combinations drawn from boundary values (negative,
// zero, odd, huge, INT64_MAX), built with the host sanitizers: any signed
// overflow, shift or out-of-bounds access in the checks aborts the run.
// Test infrastructure only.
#include <stdint.h>
#include <stdio.h>

#include "../../fp8_fine_grained_x128_amd/csrc/validate.hpp"

using namespace fp8q::check;

static uint64_t state = 1;
static uint64_t rnd() {
    uint64_t z = (state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static const int64_t kVals[] = {-1, 0, 1, 3, 16, 64, 127, 128, 129, 256, 1000, 4096, 7168, 65536, 65535LL * 512,
                                (1LL << 24) - 1, 1LL << 24, 1LL << 31, (1LL << 32), (1LL << 32) + 16, 1LL << 40,
                                1LL << 62, INT64_MAX, INT64_MIN, -128};
static int64_t v64() { return kVals[rnd() % (sizeof(kVals) / sizeof(kVals[0]))]; }
static int vint() { static const int v[] = {-1, 0, 1, 2, 3, 4, 5, 1024, 1025, 0x7fffffff}; return v[rnd() % 10]; }
static const void* vptr() {
    static const uintptr_t v[] = {0, 1u << 20, (1u << 20) + 4, (1u << 20) + 8, (1u << 20) + 2, (1u << 20) + 256};
    return reinterpret_cast<const void*>(v[rnd() % 6]);
}

static int failures = 0;
static void expect(int got, int want, const char* what) {
    if (got != want) {
        printf("FAIL %s: got %d want %d\n", what, got, want);
        ++failures;
    }
}

int main() {
    const void* P = reinterpret_cast<const void*>(uintptr_t(1) << 20);
    // fixed cases
    expect(quantize_act(P, FP8Q_BF16, 4, 128, 128, FP8Q_TILE_1x128, P, 128, P, 4, 0), kLaunch, "q_act ok");
    expect(quantize_act(P, 7, 4, 128, 128, 0, P, 128, P, 4, 0), FP8Q_EINVAL, "q_act dtype");
    expect(quantize_act(P, 1, 4, 128, 64, 0, P, 128, P, 4, 0), FP8Q_ESHAPE, "q_act ldx");
    expect(quantize_act(P, 1, 0, 128, 128, 0, nullptr, 128, nullptr, 0, 0), FP8Q_OK, "q_act empty");
    expect(quantize_act(P, 1, 4, 128, INT64_MAX, 0, P, 128, P, 4, 0), FP8Q_ESHAPE, "q_act huge ld");
    expect(gemm(P, 7168, P, 4096, P, 7168, P, 56, 0, 4096, 7168, 7168, P, FP8Q_BF16, 7168, 0, 0u), kLaunch, "gemm ok");
    expect(gemm(P, 7168, P, 4096, P, 7168, P, 56, 0, 4096, 7168, 7168, P, FP8Q_BF16, 7168, 1, 0u), FP8Q_EUNSUPPORTED,
           "gemm bf16 accumulate");
    expect(gemm(P, 7168, P, 4096, P, 7168, P, 55, 0, 4096, 7168, 7168, P, 1, 7168, 0, 0u), FP8Q_ESHAPE, "gemm ldsb");
    expect(gemm(P, 1 << 24, P, 4096, P, 7168, P, 56, 0, 4096, 7168, 7168, P, 1, 7168, 0, 0u), FP8Q_EUNSUPPORTED,
           "gemm lda 2^24");
    expect(splitk_workspace(64, nullptr, 64), FP8Q_EINVAL, "splitk null");
    expect(splitk_workspace(64, P, 60), FP8Q_ESHAPE, "splitk small");
    expect(splitk_workspace(0, nullptr, 0), kLaunch, "splitk none needed");
    expect(grouped(P, 7168, P, 32768, P, 7168, 2048LL * 7168, P, 56, 16 * 56, P, 64, 32768, 2048, 7168, P, 1, 2048,
                   0u), kLaunch, "grouped ok");
    expect(grouped(P, 7168, P, 32768, P, 7168, 2048LL * 7168 - 16, P, 56, 16 * 56, P, 64, 32768, 2048, 7168, P, 1,
                   2048, 0u), FP8Q_ESHAPE, "grouped stride");
    expect(grouped(P, 7168, P, 32768, P, 7168, INT64_MAX, P, 56, 16 * 56, P, 64, 32768, 2048, 7168, P, 1, 2048, 0u),
           FP8Q_ESHAPE, "grouped huge stride");
    expect(clock_probe(P, 0), FP8Q_ESHAPE, "probe ticks");
    // seeded sample of boundary combinations: only the sanitizers judge these
    long long launched = 0;
    for (int i = 0; i < 2000000; ++i) {
        int r = 0;
        switch (i % 9) {
            case 0: r = quantize_act(vptr(), vint(), v64(), v64(), v64(), vint(), vptr(), v64(), vptr(), v64(), vint()); break;
            case 1: r = gather_quantize_act(vptr(), vint(), v64(), v64(), v64(), vptr(), v64(), vptr(), v64(), vptr(),
                                            v64(), vint()); break;
            case 2: r = quantize_weight(vptr(), vint(), v64(), v64(), v64(), vptr(), v64(), vptr(), v64(), vint()); break;
            case 3: r = requant(vptr(), v64(), v64(), v64(), vptr(), v64(), vptr(), v64(), vptr(), v64(), vint()); break;
            case 4: r = transpose_weight(vptr(), v64(), v64(), v64(), vptr(), v64(), vptr(), v64(), vptr(), v64()); break;
            case 5: r = gemm(vptr(), v64(), vptr(), v64(), vptr(), v64(), vptr(), v64(), vint(), v64(), v64(), v64(),
                             vptr(), vint(), v64(), vint(), (unsigned)vint()); break;
            case 6: r = grouped(vptr(), v64(), vptr(), v64(), vptr(), v64(), v64(), vptr(), v64(), v64(), vptr(), vint(),
                                v64(), v64(), v64(), vptr(), vint(), v64(), (unsigned)vint()); break;
            case 7: r = splitk_workspace(v64(), vptr(), v64()); break;
            default: r = clock_probe(vptr(), v64()); break;
        }
        if (r == kLaunch) ++launched;
        if (r < kLaunch || r > FP8Q_EHIP) { printf("FAIL: status %d out of range\n", r); ++failures; }
    }
    printf("validate_driver: %d fixed-case failures; %lld of 2000000 sampled calls valid\n", failures, launched);
    return failures ? 1 : 0;
}
