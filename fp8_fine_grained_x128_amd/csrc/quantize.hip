// quantize.hip -- fine-grained FP8 quantizers for gfx950.
//
//   quantize_1x128   activations, one scale per token per 128 channels
//                    (optionally gathering rows by an index: FP8 MoE dispatch)
//   quantize_128x128 weights, one scale per 128x128 block
//   quantize_128x1   activation gradients (and requantization of cached FP8
//                    activations), one scale per channel per 128 tokens,
//                    written transposed
//
// Tile shapes: page 4 (sunipension.com, wr_id=314414), passage on Figure
// 7(a); conversion of cached activations from 1x128 to 128x1 tiles for the
// backward pass: same page and passage.  The quantization rule itself is in
// device_common.hpp.
//
// All three kernels are HBM-streaming: every input byte is read once and
// every code written once.  Tile maxima are integer maxima of magnitude bits
// (packed 16-bit for bf16 inputs), reduced inside 16-lane DPP rows and then
// through LDS.  Every kernel has a branch-free fast path, taken when the whole
// wave's tile lies inside the matrix and every scale of the wave allows the
// reciprocal quotient (the choice is wave-uniform), and a general path for
// ragged edges and tiny scales.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {

// ----------------------------------------------------------------------------
// Helpers
// ----------------------------------------------------------------------------
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load, marked non-temporal when NT: a quantizer that reads each
// input byte once need not let its input displace cached data (such as the
// codes a GEMM is about to read); measured 3-6 % faster at the step's sizes.
// A gather reads repeated source rows and keeps the normal (cached) load.
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

// Orders LDS traffic between the lanes of one wave: a wave's LDS operations
// execute in program order, the fences keep the compiler from reordering them.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bool wave_all(bool p) { return __all((int)p) != 0; }

// fl32(x/s) by the reciprocal path (valid when s >= kFastScaleMin).
__device__ __forceinline__ float quotient_fast(float x, float s, float r) {
    const float y = x * r;
    const float e = __builtin_fmaf(y, s, -x);
    return __builtin_fmaf(-e, r, y);
}

__device__ __forceinline__ uint32_t encode4_fast(float v0, float v1, float v2, float v3, float s, float r) {
    const uint32_t w = cvt2_in_range<false>(quotient_fast(v0, s, r), quotient_fast(v1, s, r), 0u);
    return cvt2_in_range<true>(quotient_fast(v2, s, r), quotient_fast(v3, s, r), w);
}

// General-path encoder of either scale rule.
template <bool POW2>
__device__ __forceinline__ uint32_t encode4_any(float v0, float v1, float v2, float v3, const TileScale& t) {
    if constexpr (POW2)
        return encode4_mul(v0, v1, v2, v3, t.r);
    else
        return encode4(v0, v1, v2, v3, t);
}

// Fast-path encoder of either scale rule (s, r of a tile whose quotient may
// take the reciprocal path).
template <bool POW2>
__device__ __forceinline__ uint32_t encode4_sr(float v0, float v1, float v2, float v3, float s, float r) {
    if constexpr (POW2)
        return encode4_mul(v0, v1, v2, v3, r);
    else
        return encode4_fast(v0, v1, v2, v3, s, r);
}

__device__ __forceinline__ TileScale scale_from(float s, float r) {
    TileScale t;
    t.s = s;
    t.r = r;
    t.fast = s >= kFastScaleMin;
    return t;
}

// Eight consecutive input elements of one row, kept in their storage form.
template <typename T>
struct Raw8;

template <>
struct Raw8<uint16_t> {  // bf16 bit patterns, two per dword
    uint4 d;
    __device__ void zero() { d = make_uint4(0, 0, 0, 0); }
    template <bool NT = true>
    __device__ void load_full(const uint16_t* p) { d = load16<NT>(p); }
    __device__ void load_partial(const uint16_t* p, int64_t n) {  // n < 8 valid elements
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < n) w[i >> 1] |= (uint32_t)p[i] << (16 * (i & 1));
        d = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ uint32_t amax_bits() const {  // fp32 bits of max |x|
        const us2 m0 = __builtin_bit_cast(us2, d.x & 0x7fff7fffu);
        const us2 m1 = __builtin_bit_cast(us2, d.y & 0x7fff7fffu);
        const us2 m2 = __builtin_bit_cast(us2, d.z & 0x7fff7fffu);
        const us2 m3 = __builtin_bit_cast(us2, d.w & 0x7fff7fffu);
        const us2 m = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                                __builtin_elementwise_max(m2, m3));
        const uint32_t mm = m[0] > m[1] ? m[0] : m[1];
        return mm << 16;
    }
    __device__ void values(float v[8]) const {
        v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
        v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
        v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
        v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
    }
};

template <>
struct Raw8<float> {
    float4 a, b;
    __device__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    template <bool NT = true>
    __device__ void load_full(const float* p) {
        const uint4 u = load16<NT>(p), v = load16<NT>(p + 4);
        a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
        b = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
    __device__ void load_partial(const float* p, int64_t n) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = i < n ? p[i] : 0.0f;
        a = make_float4(v[0], v[1], v[2], v[3]);
        b = make_float4(v[4], v[5], v[6], v[7]);
    }
    __device__ uint32_t amax_bits() const {
        uint32_t m = max(max(abs_bits(a.x), abs_bits(a.y)), max(abs_bits(a.z), abs_bits(a.w)));
        return max(m, max(max(abs_bits(b.x), abs_bits(b.y)), max(abs_bits(b.z), abs_bits(b.w))));
    }
    __device__ void values(float v[8]) const {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// Loads x[c .. c+8) of a row; elements at or beyond `valid` read as 0.
// `full` (wave-uniform) says that all 8 are valid.
template <typename T, bool NT = true>
__device__ __forceinline__ void load_row8(Raw8<T>& r, const T* row, int64_t c, int64_t valid, bool full) {
    if (full || c + 8 <= valid)
        r.template load_full<NT>(row + c);
    else if (c < valid)
        r.load_partial(row + c, valid - c);
    else
        r.zero();
}

// Stores 8 codes (two dwords) at q[c .. c+8), clipped to `valid`.
__device__ __forceinline__ void store8(uint8_t* q, int64_t c, int64_t valid, uint32_t w0, uint32_t w1) {
    if (c + 8 <= valid) {
        *reinterpret_cast<uint2*>(q + c) = make_uint2(w0, w1);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (c + i < valid) q[c + i] = (uint8_t)(((i < 4 ? w0 : w1) >> (8 * (i & 3))) & 0xffu);
    }
}

// ----------------------------------------------------------------------------
// 1x128 activation tiles.
// Work-group (a 512-column segment of a row group): W independent waves on
// W*R consecutive rows.  Segments of one row group are dispatched back to
// back, so consecutive work-groups stream whole rows (17 % more bandwidth at
// 32768x7168 bf16 than row groups first); a gather keeps row groups first,
// which lets repeated source rows hit in cache (5 % faster).  Wave w covers rows R*w ..
// R*w+R-1 of the group; lane l covers columns 8*l .. 8*l+7 of the segment, so
// a load instruction reads one row's 512 contiguous columns and each 16-lane
// DPP row holds one 128-column chunk.  Lane 16*ch + i computes the scale of
// (row i, chunk ch), stores it (one run of R rows per chunk) and passes it to
// the wave's other lanes through LDS; no work-group barrier.
// ----------------------------------------------------------------------------
// GATHER: output row r is input row gidx[r] (MoE dispatch); an index outside
// [0, rows_in) is an empty slot and quantizes as a zero row.
template <typename T, int W, int R, bool POW2, bool GATHER>
__global__ __launch_bounds__(64 * W) void quantize_1x128_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds,
    const int32_t* __restrict__ gidx, int64_t rows_in) {
    static_assert(R <= 16, "one scale per lane of a DPP row");
    __shared__ uint32_t s_amax[W][4][R];  // [wave][chunk][row]
    __shared__ float2 s_sr[W][4][R];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ch = lane >> 4;
    const int sub = lane & 15;
    // grid: x = 512-column segment, y + 65535*z = row group (x = row group,
    // y = segment for a gather)
    const int64_t seg_i = GATHER ? (int64_t)blockIdx.y : (int64_t)blockIdx.x;
    const int64_t rgrp = GATHER ? (int64_t)blockIdx.x : (int64_t)blockIdx.z * 65535 + blockIdx.y;
    if (rgrp * (W * R) >= rows) return;
    const int64_t row0 = rgrp * (W * R) + R * wave;
    const int64_t seg = seg_i * 512;
    const int64_t c = seg + 8 * lane;
    const int64_t chunk = seg_i * 4 + ch;
    const bool full_cols = seg + 512 <= cols;

    Raw8<T> raw[R];
    if (!GATHER && full_cols && row0 + R <= rows) {
        // whole tile inside the matrix: the R loads go out back to back
        // (with a branch per row they were issued one after the other)
#pragma unroll
        for (int i = 0; i < R; ++i) raw[i].template load_full<true>(x + (row0 + i) * ldx + c);
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            int64_t src = row0 + i;
            bool live = src < rows;
            if constexpr (GATHER) {
                src = live ? (int64_t)gidx[src] : -1;
                live = src >= 0 && src < rows_in;
            }
            if (live)
                load_row8<T, !GATHER>(raw[i], x + src * ldx, c, cols, full_cols);
            else
                raw[i].zero();
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t m = row_max_u32(raw[i].amax_bits());
        if (sub == 0) s_amax[wave][ch][i] = m;
    }
    wave_lds_sync();
    bool my_fast = true;
    if (sub < R) {
        const TileScale t = make_scale_mode<POW2>(s_amax[wave][ch][sub]);
        s_sr[wave][ch][sub] = make_float2(t.s, t.r);
        my_fast = t.fast;
        if (row0 + sub < rows && chunk * 128 < cols) s[chunk * lds + row0 + sub] = t.s;
    }
    wave_lds_sync();
    const bool fast = wave_all(my_fast) && full_cols && row0 + R <= rows;
    if (fast) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float2 sr = s_sr[wave][ch][i];
            float v[8];
            raw[i].values(v);
            const uint32_t w0 = encode4_sr<POW2>(v[0], v[1], v[2], v[3], sr.x, sr.y);
            const uint32_t w1 = encode4_sr<POW2>(v[4], v[5], v[6], v[7], sr.x, sr.y);
            *reinterpret_cast<uint2*>(q + (row0 + i) * ldq + c) = make_uint2(w0, w1);
        }
        return;
    }
    if (c >= cols) return;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if (row0 + i >= rows) break;
        const float2 sr = s_sr[wave][ch][i];
        const TileScale t = scale_from(sr.x, sr.y);
        float v[8];
        raw[i].values(v);
        const uint32_t w0 = encode4_any<POW2>(v[0], v[1], v[2], v[3], t);
        const uint32_t w1 = encode4_any<POW2>(v[4], v[5], v[6], v[7], t);
        store8(q + (row0 + i) * ldq, c, cols, w0, w1);
    }
}

// ----------------------------------------------------------------------------
// 128x128 weight blocks.  One work-group (8 waves) per block; wave w covers
// rows 16*w .. 16*w+15, lane l rows 4*i + l/16 (i < 4) and columns
// 8*(l%16) .. +7 (8 waves of 4 rows per lane stream 5 % faster at 7168x7168
// than 4 waves of 8 rows).  Block maximum: lanes, DPP rows, then the 32 partial maxima
// of the work-group through LDS (one barrier).  The scale is uniform over the
// work-group.
// ----------------------------------------------------------------------------
template <typename T, bool POW2>
__global__ __launch_bounds__(512) void quantize_128x128_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds) {
    __shared__ uint32_t s_part[32];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane >> 4;
    const int64_t bn = blockIdx.y, bk = blockIdx.x;
    const int64_t c = bk * 128 + 8 * (lane & 15);
    const int64_t r0 = bn * 128 + 16 * wave + sub;
    const bool full = bk * 128 + 128 <= K && bn * 128 + 128 <= N;

    Raw8<T> raw[4];
    if (full) {
        // the four loads go out back to back (a branch per row issued them
        // one after the other: 4 % slower at 7168x7168)
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i].load_full(w + (r0 + 4 * i) * ldw + c);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + 4 * i;
            if (r < N)
                load_row8(raw[i], w + r * ldw, c, K, false);
            else
                raw[i].zero();
        }
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, raw[i].amax_bits());
    m = row_max_u32(m);
    if ((lane & 15) == 0) s_part[wave * 4 + sub] = m;
    __syncthreads();
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, s_part[i]);
    const TileScale t = make_scale_mode<POW2>(amax);
    if (threadIdx.x == 0) s[bn * lds + bk] = t.s;
    if (full && t.fast) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v[8];
            raw[i].values(v);
            const uint32_t w0 = encode4_sr<POW2>(v[0], v[1], v[2], v[3], t.s, t.r);
            const uint32_t w1 = encode4_sr<POW2>(v[4], v[5], v[6], v[7], t.s, t.r);
            *reinterpret_cast<uint2*>(q + (r0 + 4 * i) * ldq + c) = make_uint2(w0, w1);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * i;
        if (r >= N) break;
        float v[8];
        raw[i].values(v);
        const uint32_t w0 = encode4_any<POW2>(v[0], v[1], v[2], v[3], t);
        const uint32_t w1 = encode4_any<POW2>(v[4], v[5], v[6], v[7], t);
        store8(q + r * ldq, c, K, w0, w1);
    }
}

// ----------------------------------------------------------------------------
// 128x1 tiles with transposed output.  A work-group handles 128 rows (tokens)
// x 128 columns (channels).  Source kinds:
//   SRC_F32 / SRC_BF16 : plain activations (the activation-gradient path),
//   SRC_FP8            : cached 1x128 codes + scales, dequantized first to
//                        v = fl32(dec(q) * s_row) (requantization).
// Thread layout while loading: 512 threads (8 waves), thread t owns channels
// 8*(t%16) .. +8 and rows 4*(t/16) .. +4.  (Against 4 waves of threads with
// 8 rows, or with 16 channels for fp8: 5-8 % more bandwidth at 8192 rows.)
// The inputs stay in registers in their storage form and are decoded twice
// (for the maxima, then for the codes), which keeps the kernel at 60-72 VGPRs.
// Column maxima: over a thread's rows, across the wave's row lanes by xor
// shuffles, then over the 4 waves through LDS; codes are transposed through a
// 128x128-byte LDS tile whose 16-byte units are XOR-swizzled by
// ((channel >> 3) & 7).  (Against decoded values held in registers and the
// maxima of all 32 row groups in LDS: 12 % more bandwidth for requantization
// and bf16 at 8192x7168, from 4 to 8 resident work-groups per CU.)
// ----------------------------------------------------------------------------
// Hides a register's value from the optimizer: values derived from it are
// recomputed after this point instead of being kept live across it.
template <typename V>
__device__ __forceinline__ void opaque(V& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
}

enum SrcKind { SRC_F32 = 0, SRC_BF16 = 1, SRC_FP8 = 2 };

__device__ __forceinline__ int swz_unit(int ch, int unit) { return unit ^ ((ch >> 3) & 7); }

template <int KIND, bool POW2>
__global__ __launch_bounds__(512) void quantize_128x1_kernel(
    const void* __restrict__ src, int64_t rows, int64_t cols, int64_t ldx,
    const float* __restrict__ s_in, int64_t lds_in,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st, int64_t ldst) {
    constexpr int kThreads = 512;
    constexpr int kWaves = kThreads / 64;
    constexpr int kCh = 8;                              // channels per thread
    constexpr int kRows = 4;                            // rows per thread
    constexpr int kChGroups = 128 / kCh;                // lanes per row
    using T = typename std::conditional<KIND == SRC_F32, float, uint16_t>::type;
    __shared__ uint32_t s_part[kWaves][128];            // per-wave column maxima
    __shared__ float2 s_sr[128];
    __shared__ __align__(16) uint8_t s_tile[128 * 128]; // [channel][token], swizzled

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int cg = t % kChGroups, rg = t / kChGroups;
    const int64_t r0 = (int64_t)blockIdx.y * 128, c0 = (int64_t)blockIdx.x * 128;
    const int64_t cbase = c0 + kCh * cg;
    const bool full = r0 + 128 <= rows && c0 + 128 <= cols;

    // The inputs stay in their storage form until they are encoded: 4 VGPRs
    // per row of 8 bf16, 2 per row of 8 codes (8 for 8 fp32), so more
    // work-groups fit.
    Raw8<T> raw[KIND == SRC_FP8 ? 1 : kRows];
    uint2 codes[KIND == SRC_FP8 ? kRows : 1];
    float rs[KIND == SRC_FP8 ? kRows : 1];
    if (full) {
        // whole tile inside the matrix: every load goes out before any
        // arithmetic (with a branch per row the loads were issued one after
        // the other: requantization 1-2 % slower at 8192x7168, bf16 2 %)
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int64_t r = r0 + kRows * rg + i;
            if constexpr (KIND == SRC_FP8) {
                codes[i] = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(src) + r * ldx + cbase);
                rs[i] = s_in[(c0 >> 7) * lds_in + r];
            } else {
                raw[i].load_full(static_cast<const T*>(src) + r * ldx + cbase);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int64_t r = r0 + kRows * rg + i;
            if constexpr (KIND == SRC_F32 || KIND == SRC_BF16) {
                if (r >= rows)
                    raw[i].zero();
                else
                    load_row8(raw[i], static_cast<const T*>(src) + r * ldx, cbase, cols, false);
            } else {
                if (r >= rows) {
                    codes[i] = make_uint2(0, 0);
                    rs[i] = 0.0f;
                    continue;
                }
                const uint8_t* row = static_cast<const uint8_t*>(src) + r * ldx;
                rs[i] = s_in[(c0 >> 7) * lds_in + r];
                if (cbase + 8 <= cols) {
                    codes[i] = *reinterpret_cast<const uint2*>(row + cbase);
                } else {
                    uint32_t wds[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        uint32_t wv = 0;
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const int64_t cc = cbase + 4 * k + b;
                            wv |= (cc < cols ? (uint32_t)row[cc] : 0u) << (8 * b);
                        }
                        wds[k] = wv;
                    }
                    codes[i] = make_uint2(wds[0], wds[1]);
                }
            }
        }
    }
    // value of channel k (0..kCh) of row i, as the quantizer sees it
    // (requantization: v = fl32(dec(q) * s_row))
    auto quad = [&](int i, int kq, float v[4]) {  // channels 4*kq .. 4*kq+3 of row i
        if constexpr (KIND == SRC_FP8) {
            const uint32_t w = kq == 0 ? codes[i].x : codes[i].y;
            float d[4];
            decode4(w, d);
#pragma unroll
            for (int b = 0; b < 4; ++b) v[b] = d[b] * rs[i];
        } else {
            float a[8];
            raw[i].values(a);
#pragma unroll
            for (int b = 0; b < 4; ++b) v[b] = a[4 * kq + b];
        }
    };
    // column maxima: per thread over its rows, across the wave's row lanes,
    // then across the 4 waves in LDS
    uint32_t m[kCh];
#pragma unroll
    for (int k = 0; k < kCh; ++k) m[k] = 0;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
#pragma unroll
        for (int kq = 0; kq < kCh / 4; ++kq) {
            if constexpr (KIND == SRC_FP8) {
                // |fl32(dec(q) * s_row)| = fl32(|dec(q)| * s_row) (s_row >= 0): the
                // magnitude comes from the multiply's source modifier, and the
                // integer maximum of non-negative fp32 bits is their maximum
                const uint32_t w = kq == 0 ? codes[i].x : codes[i].y;
                float d[4];
                decode4(w, d);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    m[4 * kq + b] = max(m[4 * kq + b], __float_as_uint(__builtin_fabsf(d[b]) * rs[i]));
                continue;
            }
            float v[4];
            quad(i, kq, v);
#pragma unroll
            for (int b = 0; b < 4; ++b) m[4 * kq + b] = max(m[4 * kq + b], abs_bits(v[b]));
        }
    }
#pragma unroll
    for (int k = 0; k < kCh; ++k) {
#pragma unroll
        for (int off = kChGroups; off < 64; off <<= 1)
            m[k] = max(m[k], (uint32_t)__shfl_xor((int)m[k], off));
    }
    if (lane < kChGroups) {
#pragma unroll
        for (int k = 0; k < kCh; ++k) s_part[wave][kCh * cg + k] = m[k];
    }
    __syncthreads();
    if (t < 128) {
        uint32_t mm = 0;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) mm = max(mm, s_part[wv][t]);
        const TileScale ts = make_scale_mode<POW2>(mm);
        s_sr[t] = make_float2(ts.s, ts.r);
        if (c0 + t < cols) st[(r0 >> 7) * ldst + c0 + t] = ts.s;
    }
    __syncthreads();
    // quantize and write codes transposed into the LDS tile (values decoded
    // again from the stored form)
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        if constexpr (KIND == SRC_FP8) {
            opaque(codes[i].x); opaque(codes[i].y);
            opaque(rs[i]);
        } else if constexpr (KIND == SRC_BF16) {
            opaque(raw[i].d.x); opaque(raw[i].d.y); opaque(raw[i].d.z); opaque(raw[i].d.w);
        }
    }
    bool my_fast = true;
#pragma unroll
    for (int k = 0; k < kCh; ++k) my_fast = my_fast && (POW2 || s_sr[kCh * cg + k].x >= kFastScaleMin);
    const bool fast = wave_all(my_fast);
    const int tok = kRows * rg;  // first token of this thread, inside 16-byte unit tok/16
#pragma unroll
    for (int kq = 0; kq < kCh / 4; ++kq) {
        float v[kRows][4];
#pragma unroll
        for (int i = 0; i < kRows; ++i) quad(i, kq, v[i]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int ch = kCh * cg + 4 * kq + b;
            const float2 sr = s_sr[ch];
            static_assert(kRows == 4, "one dword of codes per channel and thread");
            const uint32_t w0 = fast ? encode4_sr<POW2>(v[0][b], v[1][b], v[2][b], v[3][b], sr.x, sr.y)
                                     : encode4_any<POW2>(v[0][b], v[1][b], v[2][b], v[3][b], scale_from(sr.x, sr.y));
            uint8_t* p = s_tile + ch * 128 + 16 * swz_unit(ch, tok >> 4) + (tok & 15);
            *reinterpret_cast<uint32_t*>(p) = w0;
        }
    }
    __syncthreads();
    // write out: thread t -> channel 64*j + t/8, physical unit t%8
#pragma unroll
    for (int j = 0; j < 128 / (kThreads / 8); ++j) {
        const int ch = (kThreads / 8) * j + (t >> 3);
        const int unit = t & 7;
        const uint4 val = *reinterpret_cast<const uint4*>(s_tile + ch * 128 + 16 * unit);
        const int lunit = swz_unit(ch, unit);  // logical token unit held here
        const int64_t c = c0 + ch;
        const int64_t tok = r0 + 16 * lunit;
        uint8_t* dst = qt + c * ldqt + tok;
        if (full) {
            *reinterpret_cast<uint4*>(dst) = val;
            continue;
        }
        if (c >= cols) continue;
        if (tok + 16 <= rows) {
            *reinterpret_cast<uint4*>(dst) = val;
        } else {
            const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
            for (int b = 0; b < 16; ++b)
                if (tok + b < rows) dst[b] = (uint8_t)((wv[b >> 2] >> (8 * (b & 3))) & 0xffu);
        }
    }
}

// ----------------------------------------------------------------------------
// Launchers (arguments already validated by the API layer).
// ----------------------------------------------------------------------------
namespace {

template <bool GATHER>
dim3 grid_1x128(int64_t rows, int64_t cols, int rows_per_group) {
    const int64_t nrg = (rows + rows_per_group - 1) / rows_per_group, nseg = (cols + 511) / 512;
    if (GATHER) return dim3((unsigned)nrg, (unsigned)nseg);
    return dim3((unsigned)nseg, (unsigned)std::min<int64_t>(nrg, 65535), (unsigned)((nrg + 65534) / 65535));
}

template <bool POW2, bool GATHER>
void launch_1x128(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                  float* s, int64_t lds, const int32_t* gidx, int64_t rows_in, hipStream_t st) {
    // 8 waves of 2 bf16 rows (4 fp32 rows) per work-group: 3 % more bandwidth
    // at 32768x7168 bf16 than 4 waves of 4 rows.  A gather keeps 4 waves of 4
    // (8 fp32) rows: with 8 waves it ran 21 % slower.
    if (dtype == kDtypeBF16) {
        constexpr int W = GATHER ? 4 : 8, R = GATHER ? 4 : 2;
        const dim3 grid = grid_1x128<GATHER>(rows, cols, W * R);
        hipLaunchKernelGGL((quantize_1x128_kernel<uint16_t, W, R, POW2, GATHER>), grid, dim3(64 * W), 0, st,
                           static_cast<const uint16_t*>(x), rows, cols, ldx, q, ldq, s, lds, gidx, rows_in);
    } else {
        constexpr int W = GATHER ? 4 : 8, R = GATHER ? 8 : 4;
        const dim3 grid = grid_1x128<GATHER>(rows, cols, W * R);
        hipLaunchKernelGGL((quantize_1x128_kernel<float, W, R, POW2, GATHER>), grid, dim3(64 * W), 0, st,
                           static_cast<const float*>(x), rows, cols, ldx, q, ldq, s, lds, gidx, rows_in);
    }
}

template <bool POW2>
void launch_128x128(const void* w, int dtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                    float* s, int64_t lds, hipStream_t st) {
    dim3 grid((unsigned)((K + 127) / 128), (unsigned)((N + 127) / 128));
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL((quantize_128x128_kernel<uint16_t, POW2>), grid, dim3(512), 0, st,
                           static_cast<const uint16_t*>(w), N, K, ldw, q, ldq, s, lds);
    else
        hipLaunchKernelGGL((quantize_128x128_kernel<float, POW2>), grid, dim3(512), 0, st,
                           static_cast<const float*>(w), N, K, ldw, q, ldq, s, lds);
}

template <bool POW2>
void launch_128x1(const void* x, int kind, int64_t rows, int64_t cols, int64_t ldx, const float* s_in,
                  int64_t lds_in, uint8_t* qt, int64_t ldqt, float* st_out, int64_t ldst, hipStream_t st) {
    dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
    if (kind == SRC_BF16)
        hipLaunchKernelGGL((quantize_128x1_kernel<SRC_BF16, POW2>), grid, dim3(512), 0, st, x, rows, cols,
                           ldx, s_in, lds_in, qt, ldqt, st_out, ldst);
    else if (kind == SRC_F32)
        hipLaunchKernelGGL((quantize_128x1_kernel<SRC_F32, POW2>), grid, dim3(512), 0, st, x, rows, cols,
                           ldx, s_in, lds_in, qt, ldqt, st_out, ldst);
    else
        hipLaunchKernelGGL((quantize_128x1_kernel<SRC_FP8, POW2>), grid, dim3(512), 0, st, x, rows, cols,
                           ldx, s_in, lds_in, qt, ldqt, st_out, ldst);
}

}  // namespace

hipError_t launch_quantize_1x128(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, int pow2, hipStream_t st) {
    if (pow2) launch_1x128<true, false>(x, dtype, rows, cols, ldx, q, ldq, s, lds, nullptr, rows, st);
    else launch_1x128<false, false>(x, dtype, rows, cols, ldx, q, ldq, s, lds, nullptr, rows, st);
    return hipGetLastError();
}

hipError_t launch_gather_quantize_1x128(const void* x, int dtype, int64_t rows_in, int64_t cols, int64_t ldx,
                                        const int32_t* row_index, int64_t rows_out, uint8_t* q, int64_t ldq,
                                        float* s, int64_t lds, int pow2, hipStream_t st) {
    if (pow2)
        launch_1x128<true, true>(x, dtype, rows_out, cols, ldx, q, ldq, s, lds, row_index, rows_in, st);
    else
        launch_1x128<false, true>(x, dtype, rows_out, cols, ldx, q, ldq, s, lds, row_index, rows_in, st);
    return hipGetLastError();
}

hipError_t launch_quantize_128x128(const void* w, int dtype, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, float* s, int64_t lds, int pow2, hipStream_t st) {
    if (pow2) launch_128x128<true>(w, dtype, N, K, ldw, q, ldq, s, lds, st);
    else launch_128x128<false>(w, dtype, N, K, ldw, q, ldq, s, lds, st);
    return hipGetLastError();
}

hipError_t launch_quantize_128x1(const void* x, int kind, int64_t rows, int64_t cols, int64_t ldx,
                                 const float* s_in, int64_t lds_in, uint8_t* qt, int64_t ldqt,
                                 float* st_out, int64_t ldst, int pow2, hipStream_t st) {
    if (pow2) launch_128x1<true>(x, kind, rows, cols, ldx, s_in, lds_in, qt, ldqt, st_out, ldst, st);
    else launch_128x1<false>(x, kind, rows, cols, ldx, s_in, lds_in, qt, ldqt, st_out, ldst, st);
    return hipGetLastError();
}

}  // namespace fp8q
