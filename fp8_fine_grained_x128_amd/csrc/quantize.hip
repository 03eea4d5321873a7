// quantize.hip -- fine-grained FP8 quantizers for gfx950.
//
//   quantize_1x128   activations, one scale per token per 128 channels
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
// All three kernels are HBM-streaming: every input byte is read once, every
// code written once, tiles are reduced in registers (DPP within 16-lane rows)
// and LDS, and the 128x1 form transposes through an XOR-swizzled LDS tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {

// ----------------------------------------------------------------------------
// Vector input access: 8 consecutive elements of one row, widened to fp32.
// ----------------------------------------------------------------------------
template <typename T>
struct In8;

template <>
struct In8<float> {
    static constexpr int kBytes = 4;
    // Loads x[c .. c+8) of a row; elements at or beyond `valid` read as 0.
    __device__ static void load(const float* row, int64_t c, int64_t valid, float v[8]) {
        if (c + 8 <= valid) {
            float4 a = *reinterpret_cast<const float4*>(row + c);
            float4 b = *reinterpret_cast<const float4*>(row + c + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (c + i < valid) ? row[c + i] : 0.0f;
        }
    }
};

template <>
struct In8<uint16_t> {  // bf16 bit patterns
    static constexpr int kBytes = 2;
    __device__ static void load(const uint16_t* row, int64_t c, int64_t valid, float v[8]) {
        if (c + 8 <= valid) {
            uint4 a = *reinterpret_cast<const uint4*>(row + c);
            v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
            v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
            v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
            v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (c + i < valid) ? bf16_bits_to_f32(row[c + i]) : 0.0f;
        }
    }
};

__device__ __forceinline__ uint32_t amax8(const float v[8]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[i]));
    return m;
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
// Work-group: 4 waves; wave w owns 128-column chunk (4*blockIdx.y + w) of rows
// [ROWS*blockIdx.x, +ROWS).  Lane l covers row 4*i + l/16 (i < ROWS/4),
// columns 8*(l%16) .. +8 of the chunk, so one 16-lane DPP row holds one
// tile row per load.  Scales of the 64 rows of a wave are written as one
// coalesced run of s[chunk][row].
// ----------------------------------------------------------------------------
template <typename T, int ROWS>
__global__ __launch_bounds__(256) void quantize_1x128_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds) {
    static_assert(ROWS % 4 == 0 && ROWS <= 64, "rows per wave");
    constexpr int kLoads = ROWS / 4;
    __shared__ uint32_t s_amax[4][ROWS];
    __shared__ float2 s_sr[4][ROWS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t chunk = (int64_t)blockIdx.y * 4 + wave;
    const int64_t nchunks = (cols + 127) / 128;
    const bool active = chunk < nchunks;
    const int64_t row0 = (int64_t)blockIdx.x * ROWS;
    const int sub = lane >> 4;
    const int64_t c = chunk * 128 + 8 * (lane & 15);

    float v[kLoads][8];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int64_t r = row0 + 4 * i + sub;
        if (active && r < rows) {
            In8<T>::load(x + r * ldx, c, cols, v[i]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[i][k] = 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        uint32_t m = row_max_u32(amax8(v[i]));
        if ((lane & 15) == 0) s_amax[wave][4 * i + sub] = m;
    }
    __syncthreads();
    if (lane < ROWS) {
        TileScale t = make_scale(s_amax[wave][lane]);
        s_sr[wave][lane] = make_float2(t.s, t.r);
        const int64_t r = row0 + lane;
        if (active && r < rows) s[chunk * lds + r] = t.s;
    }
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int64_t r = row0 + 4 * i + sub;
        if (r >= rows) continue;
        float2 sr = s_sr[wave][4 * i + sub];
        TileScale t;
        t.s = sr.x;
        t.r = sr.y;
        t.fast = t.s >= kFastScaleMin;
        uint32_t w0 = encode4(v[i][0], v[i][1], v[i][2], v[i][3], t);
        uint32_t w1 = encode4(v[i][4], v[i][5], v[i][6], v[i][7], t);
        store8(q + r * ldq, c, cols, w0, w1);
    }
}

// ----------------------------------------------------------------------------
// 128x128 weight blocks.  One work-group (4 waves) per block; wave w covers
// rows 32*w .. +32, lane l rows 4*i + l/16 (i < 8), columns 8*(l%16) .. +8.
// ----------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quantize_128x128_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds) {
    __shared__ uint32_t s_part[16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane >> 4;
    const int64_t bn = blockIdx.y, bk = blockIdx.x;
    const int64_t c = bk * 128 + 8 * (lane & 15);

    float v[8][8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = bn * 128 + 32 * wave + 4 * i + sub;
        if (r < N) {
            In8<T>::load(w + r * ldw, c, K, v[i]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[i][k] = 0.0f;
        }
        m = max(m, amax8(v[i]));
    }
    m = row_max_u32(m);
    if ((lane & 15) == 0) s_part[wave * 4 + sub] = m;
    __syncthreads();
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, s_part[i]);
    const TileScale t = make_scale(amax);
    if (threadIdx.x == 0) s[bn * lds + bk] = t.s;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = bn * 128 + 32 * wave + 4 * i + sub;
        if (r >= N) continue;
        uint32_t w0 = encode4(v[i][0], v[i][1], v[i][2], v[i][3], t);
        uint32_t w1 = encode4(v[i][4], v[i][5], v[i][6], v[i][7], t);
        store8(q + r * ldq, c, K, w0, w1);
    }
}

// ----------------------------------------------------------------------------
// 128x1 tiles with transposed output.  A work-group handles 128 rows (tokens)
// x 128 columns (channels).  Source kinds:
//   SRC_F32 / SRC_BF16 : plain activations (the activation-gradient path),
//   SRC_FP8            : cached 1x128 codes + scales, dequantized first to
//                        v = fl32(dec(q) * s_row) (requantization).
// Thread layout while loading:
//   fp32/bf16: thread t owns channels 8*(t%16) .. +8 and rows 8*(t/16) .. +8;
//   fp8      : thread t owns channels 16*(t%8) .. +16 and rows 4*(t/8) .. +4.
// Column maxima go through LDS; codes are transposed through a 128x128-byte
// LDS tile whose 16-byte units are XOR-swizzled by ((channel >> 3) & 7).
// ----------------------------------------------------------------------------
enum SrcKind { SRC_F32 = 0, SRC_BF16 = 1, SRC_FP8 = 2 };

__device__ __forceinline__ int swz_unit(int ch, int unit) { return unit ^ ((ch >> 3) & 7); }

template <int KIND>
__global__ __launch_bounds__(256) void quantize_128x1_kernel(
    const void* __restrict__ src, int64_t rows, int64_t cols, int64_t ldx,
    const float* __restrict__ s_in, int64_t lds_in,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st, int64_t ldst) {
    constexpr int kCh = (KIND == SRC_FP8) ? 16 : 8;     // channels per thread
    constexpr int kRows = (KIND == SRC_FP8) ? 4 : 8;    // rows per thread
    constexpr int kChGroups = 128 / kCh;                // threads per row
    __shared__ uint32_t s_part[256 / kChGroups][128];   // partial column maxima
    __shared__ float2 s_sr[128];
    __shared__ __align__(16) uint8_t s_tile[128 * 128]; // [channel][token], swizzled

    const int t = threadIdx.x;
    const int cg = t % kChGroups, rg = t / kChGroups;
    const int64_t r0 = (int64_t)blockIdx.y * 128, c0 = (int64_t)blockIdx.x * 128;
    const int64_t cbase = c0 + kCh * cg;

    float v[kRows][kCh];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int64_t r = r0 + kRows * rg + i;
        if (r >= rows) {
#pragma unroll
            for (int k = 0; k < kCh; ++k) v[i][k] = 0.0f;
            continue;
        }
        if constexpr (KIND == SRC_F32) {
            In8<float>::load(static_cast<const float*>(src) + r * ldx, cbase, cols, v[i]);
        } else if constexpr (KIND == SRC_BF16) {
            In8<uint16_t>::load(static_cast<const uint16_t*>(src) + r * ldx, cbase, cols, v[i]);
        } else {
            const uint8_t* row = static_cast<const uint8_t*>(src) + r * ldx;
            const float sc = s_in[(c0 >> 7) * lds_in + r];
            uint32_t wds[4];
            if (cbase + 16 <= cols) {
                uint4 a = *reinterpret_cast<const uint4*>(row + cbase);
                wds[0] = a.x; wds[1] = a.y; wds[2] = a.z; wds[3] = a.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t wv = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int64_t cc = cbase + 4 * k + b;
                        wv |= (cc < cols ? (uint32_t)row[cc] : 0u) << (8 * b);
                    }
                    wds[k] = wv;
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float d[4];
                decode4(wds[k], d);
#pragma unroll
                for (int b = 0; b < 4; ++b) v[i][4 * k + b] = d[b] * sc;  // fl32(dec(q) * s)
            }
        }
    }
    // column maxima: per thread over its rows, then across row groups in LDS
#pragma unroll
    for (int k = 0; k < kCh; ++k) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kRows; ++i) m = max(m, abs_bits(v[i][k]));
        s_part[rg][kCh * cg + k] = m;
    }
    __syncthreads();
    if (t < 128) {
        uint32_t m = 0;
#pragma unroll
        for (int g = 0; g < 256 / kChGroups; ++g) m = max(m, s_part[g][t]);
        TileScale ts = make_scale(m);
        s_sr[t] = make_float2(ts.s, ts.r);
        if (c0 + t < cols) st[(r0 >> 7) * ldst + c0 + t] = ts.s;
    }
    __syncthreads();
    // quantize and write codes transposed into the LDS tile
#pragma unroll
    for (int k = 0; k < kCh; ++k) {
        const int ch = kCh * cg + k;
        const float2 sr = s_sr[ch];
        TileScale ts;
        ts.s = sr.x;
        ts.r = sr.y;
        ts.fast = ts.s >= kFastScaleMin;
        if constexpr (kRows == 8) {
            uint32_t w0 = encode4(v[0][k], v[1][k], v[2][k], v[3][k], ts);
            uint32_t w1 = encode4(v[4][k], v[5][k], v[6][k], v[7][k], ts);
            const int tok = 8 * rg;  // 8-byte group inside 16-byte unit tok/16
            uint8_t* p = s_tile + ch * 128 + 16 * swz_unit(ch, tok >> 4) + (tok & 15);
            *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
        } else {
            uint32_t w0 = encode4(v[0][k], v[1][k], v[2][k], v[3][k], ts);
            const int tok = 4 * rg;
            uint8_t* p = s_tile + ch * 128 + 16 * swz_unit(ch, tok >> 4) + (tok & 15);
            *reinterpret_cast<uint32_t*>(p) = w0;
        }
    }
    __syncthreads();
    // write out: thread t -> channel 32*j + t/8, physical unit t%8
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ch = 32 * j + (t >> 3);
        const int unit = t & 7;
        const uint4 val = *reinterpret_cast<const uint4*>(s_tile + ch * 128 + 16 * unit);
        const int lunit = swz_unit(ch, unit);  // logical token unit held here
        const int64_t c = c0 + ch;
        const int64_t tok = r0 + 16 * lunit;
        if (c >= cols) continue;
        uint8_t* dst = qt + c * ldqt + tok;
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
hipError_t launch_quantize_1x128(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
    const int64_t nchunks = (cols + 127) / 128;
    if (dtype == kDtypeBF16) {
        constexpr int R = 64;
        dim3 grid((unsigned)((rows + R - 1) / R), (unsigned)((nchunks + 3) / 4));
        hipLaunchKernelGGL((quantize_1x128_kernel<uint16_t, R>), grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), rows, cols, ldx, q, ldq, s, lds);
    } else {
        constexpr int R = 32;
        dim3 grid((unsigned)((rows + R - 1) / R), (unsigned)((nchunks + 3) / 4));
        hipLaunchKernelGGL((quantize_1x128_kernel<float, R>), grid, dim3(256), 0, st,
                           static_cast<const float*>(x), rows, cols, ldx, q, ldq, s, lds);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_128x128(const void* w, int dtype, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
    dim3 grid((unsigned)((K + 127) / 128), (unsigned)((N + 127) / 128));
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL(quantize_128x128_kernel<uint16_t>, grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(w), N, K, ldw, q, ldq, s, lds);
    else
        hipLaunchKernelGGL(quantize_128x128_kernel<float>, grid, dim3(256), 0, st,
                           static_cast<const float*>(w), N, K, ldw, q, ldq, s, lds);
    return hipGetLastError();
}

hipError_t launch_quantize_128x1(const void* x, int kind, int64_t rows, int64_t cols, int64_t ldx,
                                 const float* s_in, int64_t lds_in, uint8_t* qt, int64_t ldqt,
                                 float* st_out, int64_t ldst, hipStream_t st) {
    dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
    if (kind == SRC_BF16)
        hipLaunchKernelGGL(quantize_128x1_kernel<SRC_BF16>, grid, dim3(256), 0, st, x, rows, cols,
                           ldx, s_in, lds_in, qt, ldqt, st_out, ldst);
    else if (kind == SRC_F32)
        hipLaunchKernelGGL(quantize_128x1_kernel<SRC_F32>, grid, dim3(256), 0, st, x, rows, cols,
                           ldx, s_in, lds_in, qt, ldqt, st_out, ldst);
    else
        hipLaunchKernelGGL(quantize_128x1_kernel<SRC_FP8>, grid, dim3(256), 0, st, x, rows, cols,
                           ldx, s_in, lds_in, qt, ldqt, st_out, ldst);
    return hipGetLastError();
}

}  // namespace fp8q
