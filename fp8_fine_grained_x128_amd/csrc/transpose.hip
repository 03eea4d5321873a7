// transpose.hip -- exact transpose of cached FP8 weight codes and their
// 128x128 block scales, the operand layout of the Dgrad GEMM dX = dY * W.
//
// The pages run the backward GEMMs in FP8 like the forward one (page 4,
// sunipension.com wr_id=314414, passage on Figure 6).  Dgrad contracts over
// the output channels n, so W[n][k] must be read n-contiguous: Wt[k][n].
// Transposing the codes is a byte permutation and a 128x128 block holds the
// same elements in either orientation, so (codes^T, scales^T) is exactly the
// 128x128 quantization of W^T.
//
// One work-group per 128x128 tile.  Full tiles: thread t loads an 8x8 byte
// block (8 rows of 8 bytes; 16 threads cover a 128-byte row segment),
// transposes it in registers with byte permutes, and stores its 8 columns
// into a 128x128-byte LDS tile whose 8-byte slots are XOR-swizzled by the
// row's block index (conflict-free stores); 16 threads then read each output
// row's 16 slots and write 128 contiguous bytes.  Edge tiles copy byte by
// byte.  The block scale is moved by thread 0.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {

// The weight codes are read once (non-temporal loads below); the transposed
// copy is what the Dgrad GEMM reads next.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value hi:lo.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Transpose of a 4x4 byte matrix held as 4 dwords (dword r = row r, byte c =
// column c): out[c] = column c.
__device__ __forceinline__ void transpose4x4(const uint32_t a[4], uint32_t out[4]) {
    const uint32_t x0 = perm(a[1], a[0], 0x06020400u);  // a0.0 a1.0 a0.2 a1.2
    const uint32_t x1 = perm(a[1], a[0], 0x07030501u);  // a0.1 a1.1 a0.3 a1.3
    const uint32_t x2 = perm(a[3], a[2], 0x06020400u);
    const uint32_t x3 = perm(a[3], a[2], 0x07030501u);
    out[0] = perm(x2, x0, 0x05040100u);
    out[1] = perm(x3, x1, 0x05040100u);
    out[2] = perm(x2, x0, 0x07060302u);
    out[3] = perm(x3, x1, 0x07060302u);
}

__global__ __launch_bounds__(256) void transpose_weight_kernel(
    const uint8_t* __restrict__ q, int64_t N, int64_t K, int64_t ldq, const float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st, int64_t ldst) {
    __shared__ __align__(16) uint2 tile[128][16];  // [k][physical 8-byte slot of n]
    const int t = threadIdx.x;
    const int64_t bk = blockIdx.x, bn = blockIdx.y;
    const int64_t k0 = bk * 128, n0 = bn * 128;
    if (t == 0) st[bk * ldst + bn] = s[bn * lds + bk];

    if (n0 + 128 <= N && k0 + 128 <= K) {
        const int br = t >> 4, bc = t & 15;  // 8x8 block: rows n0+8br.., columns k0+8bc..
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x2 nt = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2*>(q + (n0 + 8 * br + i) * ldq + k0 + 8 * bc));
            const uint2 v = make_uint2(nt[0], nt[1]);
            lo[i] = v.x;
            hi[i] = v.y;
        }
        uint32_t c_lo0[4], c_lo1[4], c_hi0[4], c_hi1[4];
        transpose4x4(lo, c_lo0);      // columns 0..3, rows 0..3
        transpose4x4(lo + 4, c_lo1);  // columns 0..3, rows 4..7
        transpose4x4(hi, c_hi0);      // columns 4..7, rows 0..3
        transpose4x4(hi + 4, c_hi1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tile[8 * bc + j][br ^ bc] = make_uint2(c_lo0[j], c_lo1[j]);
            tile[8 * bc + 4 + j][br ^ bc] = make_uint2(c_hi0[j], c_hi1[j]);
        }
        __syncthreads();
        const int slot = t & 15;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int k = (t >> 4) + 16 * it;
            const uint2 v = tile[k][slot ^ (k >> 3)];
            *reinterpret_cast<uint2*>(qt + (k0 + k) * ldqt + n0 + 8 * slot) = v;
        }
        return;
    }
    // edge tile: element by element, consecutive threads on consecutive n
    for (int e = t; e < 128 * 128; e += 256) {
        const int64_t k = k0 + (e >> 7), n = n0 + (e & 127);
        if (k < K && n < N) qt[k * ldqt + n] = q[n * ldq + k];
    }
}

hipError_t launch_transpose_weight(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, const float* s,
                                   int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                                   hipStream_t stream) {
    dim3 grid((unsigned)((K + 127) / 128), (unsigned)((N + 127) / 128));
    hipLaunchKernelGGL(transpose_weight_kernel, grid, dim3(256), 0, stream, q, N, K, ldq, s, lds, qt, ldqt, st,
                       ldst);
    return hipGetLastError();
}

}  // namespace fp8q
