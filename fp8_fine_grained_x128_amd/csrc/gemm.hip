// gemm.hip -- block-scaled FP8 GEMM (plain and grouped) for gfx950.
//
//   C[m][n] = sum_kb  s_a(m, kb) * s_b(n, kb) * P_kb(m, n),
//   P_kb(m, n) = sum_{k in 128-wide chunk kb} dec(A[m][k]) * dec(B[n][k])
//
// Method: the matrix cores form each chunk's partial product P_kb in FP32
// and the partial is then multiplied by its two scales and added to an FP32
// running total held in vector registers (one "promotion" per 128-wide K
// interval).  Page 3 (why-be.why-be.co.kr, wr_id=55081) describes promoting
// the limited-precision matrix-unit partials to FP32 registers at a fixed K
// interval (Figure 7(b)); page 2 (xn--jj0bz6z98ct0a29q.com, wr_id=362465)
// folds dequantization into that step.  The Wgrad form (one scale per row of
// both operands per chunk) follows page 4 (sunipension.com, wr_id=314414),
// passage on Figure 6 and on 128x1 tiles.
//
// gfx950 mapping:
//   - a work-group (8 waves, 2 x 4) owns a 256x256 output tile, or a 256x448
//     strip (256x256 + 256x192 tiles) when that balances the CUs better; a
//     wave owns 128 rows x 64 columns (64 x 96 in the strip's second tile);
//   - A/B chunk tiles are copied global -> LDS with buffer_load_dwordx4 ...
//     lds (no register staging) through one buffer descriptor per operand
//     whose record count ends at the tile's last valid row, so rows past the
//     matrix read zeros with no clamping code; double-buffered, in 128-byte
//     rows whose 16-byte units are XOR-swizzled by swz(row) (below) so that
//     the fragment reads are free of LDS bank conflicts; the chunk's scales
//     travel as 4-byte direct copies (one fp32 per lane) into a small array
//     next to the tiles;
//   - default datapath: each wave converts its fragments exactly to f16 and
//     forms P_kb of every 16x16 subtile with a dependent chain of four
//     v_mfma_f32_16x16x32_f16; the promotion of a subtile's partial (four
//     FP32 FMAs per lane) is issued under the next subtile's MFMAs (the CDNA
//     analogue of the pages' two-warpgroup overlap); the codes of the next
//     row subtile are read from LDS while the current one is multiplied.
//     The FP8 and power-of-two datapaths (kMma* below) change only this
//     inner loop;
//   - the finished tile goes out through LDS as 16-byte row segments.
//
// MFMA lane layouts, checked on the hardware:
//   16x16x128 (8-bit operands): A: lane l holds row (l % 16), K bytes
//     32*(l/16) .. +32; B: lane l holds column (l % 16), the same K bytes;
//   16x16x32 (f16/bf16 operands): lane l holds row/column (l % 16), 8 values
//     of one 32-wide K step (which 8 is a free choice as long as A and B
//     agree: here K-step s of a chunk takes bytes 8s .. 8s+7 of the lane's 32);
//   D (both): lane l, element r is row 4*(l/16) + r, column (l % 16).
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copy (global_load_lds_dword): lane i's 4 bytes land
// at lds + 4 * i.  `lds` must be wave-uniform (it goes to M0).  The host
// compilation pass only parses these bodies.
__device__ __forceinline__ void copy4_to_lds(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds, 4, 0, 0);
#endif
}

// Buffer descriptor of `bytes` bytes from `base` (gfx9 raw buffer: stride 0,
// 32-bit data format).  A buffer access whose offset lies at or beyond the
// record count returns zeros instead of touching memory.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : bytes >= (int64_t)0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufferFlags);
}

// 16-byte buffer copy to LDS: lane i's bytes (at voffset + soffset from the
// descriptor's base) land at lds + 16 * i, or zeros if voffset is out of range.
__device__ __forceinline__ void buffer_copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                                     uint32_t soffset, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voffset, soffset, 0, 0);
#else
    (void)r;
    (void)voffset;
    (void)soffset;
    (void)lds;
#endif
}

// Scheduling fence: the compiler may not move instructions across it.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_barrier(0);
#endif
}

// XOR key of the 16-byte units of LDS tile row `row`: key(r) =
// 2 * (r & 3) + ((r >> 2) & 1), i.e. 0 2 4 6 1 3 5 7 for r = 0..7, repeating.
// A fragment read has lane (g = l/16, r = l%16) fetch 16 bytes of row r;
// the key was chosen by measuring the hardware bank-conflict counter for
// every XOR key linear in the row's low four bits (4096 of them, two unit
// assignments): this one reads zero conflict cycles for both halves of a
// row32 read, where keys r & 7 and (r >> 1) & 7 read 4 extra cycles per
// 16-byte read.  The key depends on r & 7 only, so it is the same function of
// the row index in the A tile and in the B tile (which starts at BM).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

struct TileCoord {
    int64_t m0;      // first row of the tile (absolute row of A / C)
    int64_t m_end;   // one past the last valid row of this tile's row range
    int64_t n0;      // first column
    int group;       // expert index (grouped GEMM) or 0
};

template <int BM, int BN, int WM, int WN, int BMODE>
struct GemmCfg {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kWaves = WM * WN;
    static constexpr int TM = BM / WM;  // wave tile rows
    static constexpr int TN = BN / WN;  // wave tile cols
    static constexpr int MT = TM / 16;
    static constexpr int NT = TN / 16;
    // B scales per chunk: a BLOCK128 tile may start at any multiple of 64
    // columns, so it touches up to ceil((64 + BN) / 128) weight blocks
    static constexpr int kNsb = BMODE == 0 ? (64 + BN + 127) / 128 : BN;
    // one B scale per 16-column subtile (ROW scales, or a wave's columns
    // that can straddle a 128-column block) instead of one per wave
    static constexpr bool kSbPerJ = BMODE == 1 || (128 % TN != 0);
    static constexpr int kSbWaves = (kNsb + 63) / 64;  // waves copying B scales
    static constexpr int kTileBytes = (BM + BN) * 128;
    static constexpr int kScaleFloats = BM + 64 * kSbWaves;
    static constexpr int kStageBytes = kTileBytes + 4 * kScaleFloats;  // tile + scales
    static constexpr int kLoadsPerWave = (BM + BN) / 8 / kWaves;  // 1 KB copies per wave
    static_assert((BM + BN) % (8 * kWaves) == 0, "tile rows must split evenly over waves");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
    static constexpr int kScaleCopies = BM / 64 + kSbWaves;  // 64-float copies per stage
    static constexpr int kScaleCopiesPerWave = (kScaleCopies + kWaves - 1) / kWaves;
    static_assert(BM % 64 == 0, "scale copies are 64 floats");
    static_assert(kStageBytes % 16 == 0, "stage alignment");
};

// Per-lane 32-bit byte offsets of the direct global->LDS copies of one tile,
// relative to the tile's base (the buffer descriptors' base).  Copy `it` of
// a wave moves the 1 KB block q = wave + kWaves * it (8 tile rows; A rows
// first, then B rows): lane l takes row 8q + l/8 and the logical 16-byte unit
// that lands at its physical unit l % 8 (the swizzle depends on the row's low
// 3 bits, which are l/8).  The offset is affine in `it` (lane offset + a
// uniform step), so the plan keeps one register per operand.  Scale copies
// clamp their index to the last valid row or block.
struct LoadPlan {
    uint32_t off_a;  // copy it = 0 of the A rows (row 8*wave + l/8)
    uint32_t off_b;  // same for the B rows
    uint32_t soff;   // scale copy (one fp32 per lane), if this wave has one
};

template <class Cfg, int BM, int BN, int BMODE>
__device__ __forceinline__ LoadPlan plan_loads(const TileCoord& tc, int64_t lda, int64_t ldb, int64_t ldsb,
                                               int64_t a_last, int64_t n_last, int wave, int lane) {
    static_assert(Cfg::kScaleCopiesPerWave == 1, "one scale copy per wave at most");
    static_assert((BM / 8) % Cfg::kWaves == 0, "A and B copies split at a copy boundary");
    LoadPlan lp;
    const int lrow = lane >> 3, unit = (lane & 7) ^ swz(lrow);
    lp.off_a = (uint32_t)((8 * wave + lrow) * lda + 16 * unit);
    lp.off_b = (uint32_t)((8 * wave + lrow) * ldb + 16 * unit);
    // scale copies: copy c < BM/64 holds s_a rows 64c .. 64c+63, the following
    // copies the B scales; copy c is issued by wave c
    const int c = wave;
    lp.soff = 0;
    if (c < BM / 64) {
        int64_t m = tc.m0 + 64 * c + lane;
        m = m < a_last ? m : a_last;
        lp.soff = (uint32_t)((m - tc.m0) * 4);
    } else if (c < Cfg::kScaleCopies) {
        const int j = 64 * (c - BM / 64) + lane;
        if (BMODE == 0) {
            int64_t nb = (tc.n0 >> 7) + (j < Cfg::kNsb ? j : Cfg::kNsb - 1);
            const int64_t nb_last = n_last >> 7;
            nb = nb < nb_last ? nb : nb_last;
            lp.soff = (uint32_t)((nb - (tc.n0 >> 7)) * ldsb * 4);
        } else {
            int64_t n = tc.n0 + j;
            n = n < n_last ? n : n_last;
            lp.soff = (uint32_t)((n - tc.n0) * 4);
        }
    }
    return lp;
}

// Issues the asynchronous copies of chunk kb (A rows, B rows and their
// scales) into one LDS stage.  `ra` / `rb` describe the tile's valid rows
// (record count = valid rows x row stride), so rows past the matrix (or past
// an expert's rows) read zeros; their results are never stored.  Copy `it`
// adds its rows' uniform offset to the lane's offset here, in one add the
// optimizer cannot see through, so that the compiler keeps one offset
// register per operand instead of hoisting one per copy out of the K loop.
// (An empty asm statement on the offsets did the same, but as they stay
// live it worked on copies of them: two more register moves per copy.
// Measured 1-2 % faster across the GEMMs without them.)
// (Only copies first .. last-1 of the wave; the scale copy goes with copy 0.)
template <class Cfg, int BM, int BMODE>
__device__ __forceinline__ void load_stage(uint8_t* lds_tile, float* lds_scale, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, const float* sa_tile,
                                           const float* sb_tile, int64_t lda, int64_t ldb, int64_t ldsa,
                                           int64_t ldsb, const LoadPlan& lp, int64_t kb, int wave,
                                           int first = 0, int last = Cfg::kLoadsPerWave) {
    constexpr int kStep = 8 * Cfg::kWaves;  // rows between consecutive copies of a wave
    const uint32_t oa = lp.off_a, ob = lp.off_b;
    const uint32_t kofs = (uint32_t)kb * 128u;
#pragma unroll
    for (int it = 0; it < Cfg::kLoadsPerWave; ++it) {
        if (it < first || it >= last) continue;  // constant after inlining
        const int q = wave + Cfg::kWaves * it;
        const bool is_a = it < (BM / 8) / Cfg::kWaves;
        const int rel = is_a ? kStep * it : kStep * it - BM;  // first row of this copy's block minus 8*wave
        const uint32_t step = (uint32_t)(rel * (is_a ? lda : ldb));  // uniform
        uint32_t voff;
        asm volatile("v_add_u32 %0, %1, %2" : "=v"(voff) : "s"(step), "v"(is_a ? oa : ob));
        buffer_copy16_to_lds(is_a ? ra : rb, voff, kofs, lds_tile + 1024 * q);
    }
    if (first != 0) return;
    const int c = wave;
    if (c < BM / 64) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(sa_tile + kb * ldsa);
        copy4_to_lds(base + lp.soff, lds_scale + 64 * c);
    } else if (c < Cfg::kScaleCopies) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(BMODE == 0 ? sb_tile + kb : sb_tile + kb * ldsb);
        copy4_to_lds(base + lp.soff, lds_scale + 64 * c);
    }
}

// Matrix-core datapath of the chunk partials.
//   kMmaF16 : codes are converted exactly to f16 (every E4M3 value is an f16
//             value) and multiplied by v_mfma_f32_16x16x32_f16, whose products
//             are exact and whose sums round like FP32 additions.  This meets
//             the 1e-5 * sum|a*b| * s_a * s_b bound.
//   kMmaFp8 : v_mfma_f32_16x16x128_f8f6f4 on the codes directly, twice the
//             matrix-core rate, but the instruction adds each run of 8
//             adjacent products with an alignment window of about 14 bit
//             positions below the largest of them (smaller bits are dropped),
//             the same kind of limited accumulation that the pages report for
//             FP8 tensor cores; promotion every 128 bounds its growth but the
//             per-instruction loss can exceed the bound above.
//   kMmaBf16Fold / kMmaFp8Scaled : power-of-two scales only (the operands
//             of the power-of-two quantizers).  A scale 2^e is then exact in
//             any format with an 8-bit exponent, so it moves into the
//             operands and the matrix core accumulates the whole K with no
//             promotion step:
//               kMmaBf16Fold : v_cvt_scalef32_pk_bf16_fp8 forms dec(q) * 2^e
//                 exactly as bf16 (the conversion uses the exponent of its
//                 scale operand, which is all a power of two has; checked on
//                 the hardware for every code and every e in [-127, 127]),
//                 and v_mfma_f32_16x16x32_bf16 adds exact products like FP32;
//               kMmaFp8Scaled : v_mfma_scale_f32_16x16x128_f8f6f4 with each
//                 lane's E8M0 scale (the fp32 exponent field of 2^e) applied
//                 by the hardware to the 32 K values of its row or column,
//                 at the FP8 matrix rate; the in-instruction run-of-8
//                 truncation of kMmaFp8 applies, the accumulator adds like
//                 FP32.
static_assert(kMmaF16 == 0 && kMmaFp8 == 1 && kMmaBf16Fold == 2 && kMmaFp8Scaled == 3,
              "datapath ids (launch.hpp)");

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Two E4M3 codes (byte pair WORD of w) -> two f16 values, exact (scale 1).
template <bool WORD>
__device__ __forceinline__ v2h e4m3x2_to_f16(uint32_t w) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, WORD);
#else
    (void)w;
    return v2h{};
#endif
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two E4M3 codes times the power-of-two scale `s` -> two bf16 values (exact
// while the product stays in the bf16 range).
template <bool WORD>
__device__ __forceinline__ v2bf e4m3x2_to_bf16_scaled(uint32_t w, float s) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, WORD);
#else
    (void)w;
    (void)s;
    return v2bf{};
#endif
}

__device__ __forceinline__ v8bf e4m3x8_to_bf16_scaled(uint32_t w0, uint32_t w1, float s) {
    const v2bf a = e4m3x2_to_bf16_scaled<false>(w0, s), b = e4m3x2_to_bf16_scaled<true>(w0, s);
    const v2bf c = e4m3x2_to_bf16_scaled<false>(w1, s), d = e4m3x2_to_bf16_scaled<true>(w1, s);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E8M0 code of a power-of-two fp32 scale: its exponent field (2^-127, stored
// as an fp32 subnormal, and 0 both give code 0 = 2^-127).
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }

// Eight codes (two dwords) -> one f16 MFMA operand.
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
    const v2h a = e4m3x2_to_f16<false>(w0), b = e4m3x2_to_f16<true>(w0);
    const v2h c = e4m3x2_to_f16<false>(w1), d = e4m3x2_to_f16<true>(w1);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's 32 codes of one tile row for the chunk: logical 16-byte units 2g
// and 2g+1 of the row (g = lane / 16), read from their swizzled positions.
__device__ __forceinline__ void read_row32(const uint8_t* rows, int row, int g, uint4& lo, uint4& hi) {
    const uint8_t* base = rows + row * 128;
    lo = *reinterpret_cast<const uint4*>(base + 16 * ((2 * g) ^ swz(row)));
    hi = *reinterpret_cast<const uint4*>(base + 16 * ((2 * g + 1) ^ swz(row)));
}

// f16 datapath of one chunk.  Pipelined over the (i, j) steps: the four
// K-step MFMAs of a 16x16 subtile are one dependent chain (they issue back to
// back), and the partial of step s is promoted during step s+2, a whole step
// after its last MFMA, so its promotion FMAs neither stall on the result nor
// need hazard waits.  (Promotion during step s+1 needed 23 seven-cycle hazard
// waits per chunk; with the A codes read a whole subtile ahead, which the
// registers allowed there, it ran 2.8 % slower.)  The next row subtile's codes
// are read during the second-to-last step of the current one.
// Promotion factors: JS >= 0 (BLOCK128 scales): subtiles j < JS lie in the
// wave's first 128-column weight block (scale sb[0]), the others in the next
// one (sb[1]); both products s_a * s_b are formed once per row subtile, so the
// promotion is one FMA per element.  JS < 0 (ROW scales, or a wave tile that
// crosses a block inside a subtile): s_a once per row subtile, times sb[j]
// per element.
template <class Cfg, int BM, int JS, class Issue>
__device__ __forceinline__ void chunk_f16(const uint8_t* As, const uint8_t* Bs, const float* lds_scale,
                                          const float* sb, v4f (&acc)[Cfg::MT][Cfg::NT], int wm, int wn,
                                          int g, int r16, Issue&& issue) {
    // The next chunk's copies go out one per step over the first steps
    // instead of all before the first one: eight waves issuing eight 1 KB
    // copies each at once queue at the compute unit's texture address unit,
    // and a wave stalled there issues no MFMA.  (Measured: 1-5 % faster
    // across the GEMMs; one copy every 2, 3 or 4 steps was no better.)
    // Wave tiles of at most 64 rows issue them all in the first step (below).
    constexpr int kParts = Cfg::kLoadsPerWave;
    constexpr int kSteps = Cfg::MT * Cfg::NT;
    constexpr int kIssueStride = 1;
    constexpr bool kTwo = JS >= 0;
    constexpr bool kHi = kTwo && JS < Cfg::NT;  // some subtiles use the second block
    // B column subtiles are read and converted during the first row of steps
    // (i = 0): step j reads the codes of subtile j + kAhead and, after its
    // MFMAs, converts subtile j + 1, so a chunk's first MFMA waits for two
    // LDS reads and 32 conversions per wave instead of all NT subtiles'.
    // (Measured 0.5-1.5 % faster across the GEMMs; reading two steps ahead
    // was no better.)
    constexpr int kAhead = 1;
    v8h bf[Cfg::NT][4];
    uint4 blo[Cfg::NT], bhi[Cfg::NT];
    auto read_b = [&](int j) __attribute__((always_inline)) {
        read_row32(Bs, wn * Cfg::TN + 16 * j + r16, g, blo[j], bhi[j]);
    };
    auto convert_b = [&](int j) __attribute__((always_inline)) {
        bf[j][0] = e4m3x8_to_f16(blo[j].x, blo[j].y);
        bf[j][1] = e4m3x8_to_f16(blo[j].z, blo[j].w);
        bf[j][2] = e4m3x8_to_f16(bhi[j].x, bhi[j].y);
        bf[j][3] = e4m3x8_to_f16(bhi[j].z, bhi[j].w);
    };
    read_b(0);
    static_assert(Cfg::NT >= 2, "promotion two steps behind");
    // factors of subtile i (sf, sf2) and of subtile i-1 (sfo, sf2o)
    float4 sf = {0.0f, 0.0f, 0.0f, 0.0f}, sf2 = sf, sfo = sf, sf2o = sf, sa_pend = sf;
    v4f p1 = {0.0f, 0.0f, 0.0f, 0.0f}, p2 = p1;  // partials of steps s-1 and s-2
    auto promote = [&](int pi, int pj, const v4f& pp, bool old) {
        if constexpr (kTwo) {
            const float4 f = (!kHi || pj < JS) ? (old ? sfo : sf) : (old ? sf2o : sf2);
            acc[pi][pj][0] = __builtin_fmaf(pp[0], f.x, acc[pi][pj][0]);
            acc[pi][pj][1] = __builtin_fmaf(pp[1], f.y, acc[pi][pj][1]);
            acc[pi][pj][2] = __builtin_fmaf(pp[2], f.z, acc[pi][pj][2]);
            acc[pi][pj][3] = __builtin_fmaf(pp[3], f.w, acc[pi][pj][3]);
        } else {
            const float s = sb[pj];
            const float4 f = old ? sfo : sf;
            acc[pi][pj][0] = __builtin_fmaf(pp[0], f.x * s, acc[pi][pj][0]);
            acc[pi][pj][1] = __builtin_fmaf(pp[1], f.y * s, acc[pi][pj][1]);
            acc[pi][pj][2] = __builtin_fmaf(pp[2], f.z * s, acc[pi][pj][2]);
            acc[pi][pj][3] = __builtin_fmaf(pp[3], f.w * s, acc[pi][pj][3]);
        }
    };
    uint4 rlo, rhi;  // codes of the next row subtile
    read_row32(As, wm * Cfg::TM + r16, g, rlo, rhi);
#pragma unroll
    for (int j = 1; j < kAhead && j < Cfg::NT; ++j) read_b(j);
    convert_b(0);
#pragma unroll
    for (int i = 0; i < Cfg::MT; ++i) {
        v8h af[4];
        af[0] = e4m3x8_to_f16(rlo.x, rlo.y);
        af[1] = e4m3x8_to_f16(rlo.z, rlo.w);
        af[2] = e4m3x8_to_f16(rhi.x, rhi.y);
        af[3] = e4m3x8_to_f16(rhi.z, rhi.w);
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) {
            if (i == 0 && j + kAhead < Cfg::NT) read_b(j + kAhead);
            v4f p = {0.0f, 0.0f, 0.0f, 0.0f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[0], bf[j][0], p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[1], bf[j][1], p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[2], bf[j][2], p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[3], bf[j][3], p, 0, 0, 0);
            if (i == 0 && j + 1 < Cfg::NT) convert_b(j + 1);
            if (j == 0) {  // s_a of subtile i; the factors of i-1 stay for two more steps
                sa_pend = *reinterpret_cast<const float4*>(lds_scale + wm * Cfg::TM + 16 * i + 4 * g);
                sfo = sf;
                sf2o = sf2;
            }
            if (j == 1) {  // factors of subtile i, first used in step j = 2
                if constexpr (kTwo) {
                    sf = make_float4(sa_pend.x * sb[0], sa_pend.y * sb[0], sa_pend.z * sb[0], sa_pend.w * sb[0]);
                    if constexpr (kHi)
                        sf2 = make_float4(sa_pend.x * sb[1], sa_pend.y * sb[1], sa_pend.z * sb[1], sa_pend.w * sb[1]);
                } else {
                    sf = sa_pend;
                }
            }
            const int s = i * Cfg::NT + j;
            if constexpr (Cfg::MT <= 4) {
                // wave tiles of at most 64 rows: a chunk is short, and copies
                // going out one per step land too late for the next one, so
                // they all go out in step 0 (the grouped GEMM's 64- and
                // 128-row tiles, whose B rows stream from HBM: 1.3 % faster
                // over the grouped workload; no change on the strip
                // kernel's 64-row-wave second tile)
                if (s == 0) {
#pragma unroll
                    for (int part = 0; part < kParts; ++part) issue(part);
                }
            } else if (s % kIssueStride == 0 && s / kIssueStride < kParts) {
                issue(s / kIssueStride);
            }
            if (s >= 2) {  // step s-2: its MFMAs finished a whole step ago
                const int pi = (s - 2) / Cfg::NT, pj = (s - 2) % Cfg::NT;
                promote(pi, pj, p2, pi != i);
            }
            if (j == Cfg::NT - 2 && i + 1 < Cfg::MT) read_row32(As, wm * Cfg::TM + 16 * (i + 1) + r16, g, rlo, rhi);
            p2 = p1;
            p1 = p;
            // keep steps in program order: the scheduler interleaves the
            // MFMAs and VALU work of one step, but hoisting later steps
            // would keep several partials and fragments live at once
            sched_fence();
        }
    }
    constexpr int S = Cfg::MT * Cfg::NT;
    promote((S - 2) / Cfg::NT, (S - 2) % Cfg::NT, p2, false);
    promote(Cfg::MT - 1, Cfg::NT - 1, p1, false);
    static_assert((kSteps + kIssueStride - 1) / kIssueStride >= kParts, "every copy is issued inside the steps");
}

// One 128-wide chunk on one LDS stage: matrix-core partials + promotion.
// f16 datapath: K-step s (0..3) of a lane uses bytes 8s .. 8s+7 of its 32
// codes, for A and B alike, so every k of the chunk meets its partner once.
// ncol: the wave's first column counted from the first 128-column block
// whose scale the stage holds ((n0 & 127) + wn * TN; used for BLOCK128).
// JS (f16 datapath, BLOCK128 scales): the subtile at which this wave's
// columns enter the next 128-column weight block, when the caller knows it
// (-2: not known; a crossing is then handled per subtile).
// issue(part) issues copy `part` of the next chunk's stage (0 .. kLoadsPerWave-1).
template <class Cfg, int BM, int BMODE, int MMA, int JS = -2, class Issue>
__device__ __forceinline__ void compute_chunk(const uint8_t* lds_tile, const float* lds_scale,
                                              v4f (&acc)[Cfg::MT][Cfg::NT], int wm, int wn,
                                              int lane, int ncol, Issue&& issue) {
    if constexpr (MMA != kMmaF16) {
#pragma unroll
        for (int part = 0; part < Cfg::kLoadsPerWave; ++part) issue(part);
    }
    const uint8_t* As = lds_tile;
    const uint8_t* Bs = lds_tile + BM * 128;
    const int g = lane >> 4;
    const int r16 = lane & 15;

    constexpr bool kPerJ = Cfg::kSbPerJ;
    float sbv[kPerJ ? Cfg::NT : 1];
    if constexpr (BMODE == 0) {
        if constexpr (kPerJ) {
#pragma unroll
            for (int j = 0; j < Cfg::NT; ++j) sbv[j] = lds_scale[BM + ((ncol + 16 * j) >> 7)];
        } else {
            sbv[0] = lds_scale[BM + (ncol >> 7)];
        }
    } else {
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) sbv[j] = lds_scale[BM + wn * Cfg::TN + 16 * j + r16];
    }

    if constexpr (MMA == kMmaF16) {
        if constexpr (BMODE == 0 && !kPerJ) {
            chunk_f16<Cfg, BM, Cfg::NT>(As, Bs, lds_scale, sbv, acc, wm, wn, g, r16, issue);
        } else if constexpr (BMODE == 0 && JS >= 0) {
            // the caller found this wave's block boundary at subtile JS
            float sb2[2];
            sb2[0] = lds_scale[BM + (ncol >> 7)];
            sb2[1] = JS < Cfg::NT ? lds_scale[BM + (ncol >> 7) + 1] : sb2[0];
            chunk_f16<Cfg, BM, JS>(As, Bs, lds_scale, sb2, acc, wm, wn, g, r16, issue);
        } else {
            chunk_f16<Cfg, BM, -1>(As, Bs, lds_scale, sbv, acc, wm, wn, g, r16, issue);
        }
    } else if constexpr (MMA == kMmaBf16Fold) {
        v8bf bf[Cfg::NT][4];
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) {
            uint4 lo, hi;
            read_row32(Bs, wn * Cfg::TN + 16 * j + r16, g, lo, hi);
            const float sb = kPerJ ? sbv[kPerJ ? j : 0] : sbv[0];
            bf[j][0] = e4m3x8_to_bf16_scaled(lo.x, lo.y, sb);
            bf[j][1] = e4m3x8_to_bf16_scaled(lo.z, lo.w, sb);
            bf[j][2] = e4m3x8_to_bf16_scaled(hi.x, hi.y, sb);
            bf[j][3] = e4m3x8_to_bf16_scaled(hi.z, hi.w, sb);
        }
#pragma unroll
        for (int i = 0; i < Cfg::MT; ++i) {
            uint4 lo, hi;
            read_row32(As, wm * Cfg::TM + 16 * i + r16, g, lo, hi);
            const float sa = lds_scale[wm * Cfg::TM + 16 * i + r16];  // this lane's A row
            v8bf af[4];
            af[0] = e4m3x8_to_bf16_scaled(lo.x, lo.y, sa);
            af[1] = e4m3x8_to_bf16_scaled(lo.z, lo.w, sa);
            af[2] = e4m3x8_to_bf16_scaled(hi.x, hi.y, sa);
            af[3] = e4m3x8_to_bf16_scaled(hi.z, hi.w, sa);
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int j = 0; j < Cfg::NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st], bf[j][st], acc[i][j], 0, 0, 0);
        }
    } else if constexpr (MMA == kMmaFp8Scaled) {
        v8i bfr[Cfg::NT];
        int sbe[Cfg::NT];
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) {
            uint4 lo, hi;
            read_row32(Bs, wn * Cfg::TN + 16 * j + r16, g, lo, hi);
            bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sbe[j] = e8m0_of(kPerJ ? sbv[kPerJ ? j : 0] : sbv[0]);
        }
        uint4 lo, hi;
        read_row32(As, wm * Cfg::TM + r16, g, lo, hi);
        float sa_next = lds_scale[wm * Cfg::TM + r16];
#pragma unroll
        for (int i = 0; i < Cfg::MT; ++i) {
            const v8i afr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int sae = e8m0_of(sa_next);
            if (i + 1 < Cfg::MT) {
                read_row32(As, wm * Cfg::TM + 16 * (i + 1) + r16, g, lo, hi);
                sa_next = lds_scale[wm * Cfg::TM + 16 * (i + 1) + r16];
            }
#pragma unroll
            for (int j = 0; j < Cfg::NT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr[j], acc[i][j], 0, 0, 0, sae, 0,
                                                                            sbe[j]);
        }
    } else {
        v8i bfr[Cfg::NT];
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) {
            uint4 lo, hi;
            read_row32(Bs, wn * Cfg::TN + 16 * j + r16, g, lo, hi);
            bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        // One MFMA per (i, j) step forms the chunk's partial; as in the f16
        // datapath it is promoted two steps later, when the MFMA has long
        // finished (promoting right after the MFMA stalled on its result:
        // 5.7 % slower), and the next row subtile's codes are read during the
        // second-to-last step.
        float4 sf = {0.0f, 0.0f, 0.0f, 0.0f}, sfo = sf;  // s_a of subtiles i and i-1
        v4f p1 = {0.0f, 0.0f, 0.0f, 0.0f}, p2 = p1;       // partials of steps s-1, s-2
        auto promote = [&](int pi, int pj, const v4f& pp, bool old) {
            const float4 f = old ? sfo : sf;
            const float sb = kPerJ ? sbv[kPerJ ? pj : 0] : sbv[0];
            acc[pi][pj][0] = __builtin_fmaf(pp[0], f.x * sb, acc[pi][pj][0]);
            acc[pi][pj][1] = __builtin_fmaf(pp[1], f.y * sb, acc[pi][pj][1]);
            acc[pi][pj][2] = __builtin_fmaf(pp[2], f.z * sb, acc[pi][pj][2]);
            acc[pi][pj][3] = __builtin_fmaf(pp[3], f.w * sb, acc[pi][pj][3]);
        };
        uint4 lo, hi;
        read_row32(As, wm * Cfg::TM + r16, g, lo, hi);
#pragma unroll
        for (int i = 0; i < Cfg::MT; ++i) {
            const v8i afr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
            for (int j = 0; j < Cfg::NT; ++j) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr[j], zero, 0, 0, 0, 0, 0, 0);
                if (j == 0) {
                    sfo = sf;
                    sf = *reinterpret_cast<const float4*>(lds_scale + wm * Cfg::TM + 16 * i + 4 * g);
                }
                const int s = i * Cfg::NT + j;
                if (s >= 2) {
                    const int pi = (s - 2) / Cfg::NT, pj = (s - 2) % Cfg::NT;
                    promote(pi, pj, p2, pi != i);
                }
                if (j == Cfg::NT - 2 && i + 1 < Cfg::MT) read_row32(As, wm * Cfg::TM + 16 * (i + 1) + r16, g, lo, hi);
                p2 = p1;
                p1 = p;
                sched_fence();
            }
        }
        constexpr int S = Cfg::MT * Cfg::NT;
        promote((S - 2) / Cfg::NT, (S - 2) % Cfg::NT, p2, false);
        promote(Cfg::MT - 1, Cfg::NT - 1, p1, false);
    }
}

template <class Cfg, int OUT, bool ACC>
__device__ __forceinline__ void store_tile(const v4f (&acc)[Cfg::MT][Cfg::NT], void* c, int64_t ldc,
                                           const TileCoord& tc, int64_t N, int wm, int wn,
                                           int lane) {
    const int g = lane >> 4;
    const int r16 = lane & 15;
#pragma unroll
    for (int i = 0; i < Cfg::MT; ++i) {
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) {
            const int64_t n = tc.n0 + wn * Cfg::TN + 16 * j + r16;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = tc.m0 + wm * Cfg::TM + 16 * i + 4 * g + r;
                if (m >= tc.m_end) continue;
                if constexpr (OUT == kDtypeF32) {
                    float* p = static_cast<float*>(c) + m * ldc + n;
                    if constexpr (ACC)
                        *p = *p + acc[i][j][r];
                    else
                        *p = acc[i][j][r];
                } else {
                    uint16_t* p = static_cast<uint16_t*>(c) + m * ldc + n;
                    *p = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

// Output through LDS: each wave writes its tile into a private LDS region
// (row pitch = row bytes + 16, which keeps the four rows of an accumulator
// write in distinct banks), then stores 16-byte row segments, so a global
// store instruction writes whole row pieces instead of one element per lane.
// RP rows of the wave tile per pass.  Requires c and ldc * element size to be
// 16-byte aligned (checked by the host); columns past N fall back to
// element stores.  `region`: this wave's LDS bytes (at least RP * pitch).
template <class Cfg, int OUT, bool ACC>
__device__ __forceinline__ void store_tile_vec(const v4f (&acc)[Cfg::MT][Cfg::NT], void* c, int64_t ldc,
                                               const TileCoord& tc, int64_t N, int wm, int wn, int lane,
                                               uint8_t* region) {
    constexpr int kEl = OUT == kDtypeF32 ? 4 : 2;       // bytes per output element
    constexpr int kRowBytes = Cfg::TN * kEl;
    constexpr int kUnits = kRowBytes / 16;               // 16-byte units per row
    constexpr int kPerUnit = 16 / kEl;                   // elements per unit
    constexpr int kPitch = kRowBytes + 16;
    constexpr int RP = OUT == kDtypeF32 || Cfg::TM % 64 != 0 ? 32 : 64;  // rows per pass
    static_assert(kRowBytes % 16 == 0 && Cfg::TM % RP == 0 && RP % 16 == 0, "store tiling");
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int64_t n_base = tc.n0 + wn * Cfg::TN;
#pragma unroll
    for (int pass = 0; pass < Cfg::TM / RP; ++pass) {
        if (pass > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the last pass are done
#pragma unroll
        for (int ii = 0; ii < RP / 16; ++ii) {
            const int i = pass * (RP / 16) + ii;
#pragma unroll
            for (int j = 0; j < Cfg::NT; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint8_t* dst = region + (16 * ii + 4 * g + r) * kPitch + (16 * j + r16) * kEl;
                    if constexpr (OUT == kDtypeF32)
                        *reinterpret_cast<float*>(dst) = acc[i][j][r];
                    else
                        *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's writes are visible to its reads
#pragma unroll
        for (int idx0 = 0; idx0 < RP * kUnits; idx0 += 64) {
            const int idx = idx0 + lane;
            if (RP * kUnits % 64 != 0 && idx >= RP * kUnits) break;
            const int row = idx / kUnits, unit = idx % kUnits;
            const int64_t m = tc.m0 + wm * Cfg::TM + pass * RP + row;
            if (m >= tc.m_end) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(region + row * kPitch + unit * 16);
            const int64_t n = n_base + unit * kPerUnit;
            uint8_t* gp = static_cast<uint8_t*>(c) + (m * ldc + n) * kEl;
            if (n + kPerUnit <= N) {
                if constexpr (ACC) {
                    const float4 o = *reinterpret_cast<const float4*>(gp);
                    float4 w;
                    w.x = o.x + __uint_as_float(v.x);
                    w.y = o.y + __uint_as_float(v.y);
                    w.z = o.z + __uint_as_float(v.z);
                    w.w = o.w + __uint_as_float(v.w);
                    *reinterpret_cast<float4*>(gp) = w;
                } else {
                    *reinterpret_cast<uint4*>(gp) = v;
                }
            } else {
                const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < kPerUnit; ++e) {
                    if (n + e >= N) break;
                    if constexpr (OUT == kDtypeF32) {
                        float* q = reinterpret_cast<float*>(gp) + e;
                        if constexpr (ACC)
                            *q = *q + __uint_as_float(wv[e]);
                        else
                            *q = __uint_as_float(wv[e]);
                    } else {
                        reinterpret_cast<uint16_t*>(gp)[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
    }
}

struct GemmParams {
    const uint8_t* a;
    int64_t lda;
    const float* sa;
    int64_t ldsa;
    const uint8_t* b;
    int64_t ldb;
    int64_t b_group_stride;
    const float* sb;
    int64_t ldsb;
    int64_t sb_group_stride;
    const int32_t* offsets;
    int groups;
    int64_t M, N, K;
    void* c;
    int64_t ldc;
    int64_t tiles_m, tiles_n;  // plain GEMM tile grid
    int vec_store;             // c and ldc allow 16-byte stores
    // split K (plain GEMM): slice s covers chunks [s * kb_split, (s+1) * kb_split)
    // and writes its FP32 partial tile to ws + s * ws_stride (row stride ldws)
    int splits;
    int64_t kb_split;
    float* ws;
    int64_t ldws;
    int64_t ws_stride;
};

// Full K loop for one output tile.  Two LDS stages: while chunk kb is
// computed from stage kb&1, the copies of chunk kb+1 land in the other stage;
// one wait + barrier per chunk.
template <int BM, int BN, int WM, int WN, int BMODE, int OUT, bool ACC, int MMA, int JS = -2,
          bool kPerTileLane = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const TileCoord& tc,
                                          const uint8_t* __restrict__ b, const float* __restrict__ sb,
                                          uint8_t* lds, int64_t kb0 = 0, int64_t kb1 = -1,
                                          void* c_out = nullptr, int64_t ldc_out = 0) {
    using Cfg = GemmCfg<BM, BN, WM, WN, BMODE>;
    // kPerTileLane (persistent tile loops): threadIdx.x is made opaque to the
    // optimizer, so the per-lane constants derived from it are formed per
    // tile instead of hoisted out of the tile loop (where they would be held
    // across every K loop and spilled).
    int t = threadIdx.x;
    if constexpr (kPerTileLane) asm volatile("" : "+v"(t));
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t a_last = tc.m_end - 1;  // clamp target for rows past the range
    const int64_t n_last = p.N - 1;
    const int64_t nk = kb1 < 0 ? p.K / 128 : kb1;  // one past the last chunk of this tile's K range
    void* const c = c_out ? c_out : p.c;
    const int64_t ldc = c_out ? ldc_out : p.ldc;

    const uint8_t* a_tile = p.a + tc.m0 * p.lda;
    const uint8_t* b_tile = b + tc.n0 * p.ldb;
    const float* sa_tile = p.sa + tc.m0;
    const float* sb_tile = BMODE == 0 ? sb + (tc.n0 >> 7) * p.ldsb : sb + tc.n0;
    const LoadPlan lp = plan_loads<Cfg, BM, BN, BMODE>(tc, p.lda, p.ldb, p.ldsb, a_last, n_last, wave, lane);
    const int64_t a_rows = tc.m_end - tc.m0, b_rows = p.N - tc.n0;  // valid rows from the tile start
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_tile, a_rows * p.lda);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_tile, b_rows * p.ldb);
    const int ncol = (int)(tc.n0 & 127) + wn * Cfg::TN;

    v4f acc[Cfg::MT][Cfg::NT];
#pragma unroll
    for (int i = 0; i < Cfg::MT; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::NT; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    load_stage<Cfg, BM, BMODE>(lds + (kb0 & 1) * Cfg::kStageBytes,
                               reinterpret_cast<float*>(lds + (kb0 & 1) * Cfg::kStageBytes + Cfg::kTileBytes), ra,
                               rb, sa_tile, sb_tile, p.lda, p.ldb, p.ldsa, p.ldsb, lp, kb0, wave);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int64_t kb = kb0; kb < nk; ++kb) {
        uint8_t* cur = lds + (kb & 1) * Cfg::kStageBytes;
        uint8_t* nxt = lds + ((kb + 1) & 1) * Cfg::kStageBytes;
        // branch-free: after the last chunk the copies fetch chunk kb again
        // into the stage that is not read any more
        const int64_t kb_next = kb + 1 < nk ? kb + 1 : kb;
        auto issue = [&](int part) __attribute__((always_inline)) {
            load_stage<Cfg, BM, BMODE>(nxt, reinterpret_cast<float*>(nxt + Cfg::kTileBytes), ra, rb, sa_tile,
                                       sb_tile, p.lda, p.ldb, p.ldsa, p.ldsb, lp, kb_next, wave, part, part + 1);
        };
        compute_chunk<Cfg, BM, BMODE, MMA, JS>(cur, reinterpret_cast<const float*>(cur + Cfg::kTileBytes), acc,
                                               wm, wn, lane, ncol, issue);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    if (c_out || p.vec_store) {  // split partials: 256-byte aligned, row stride a multiple of 4
        constexpr int kRegion = (2 * Cfg::kStageBytes / Cfg::kWaves) & ~15;
        store_tile_vec<Cfg, OUT, ACC>(acc, c, ldc, tc, p.N, wm, wn, lane, lds + wave * kRegion);
    } else {
        store_tile<Cfg, OUT, ACC>(acc, c, ldc, tc, p.N, wm, wn, lane);
    }
}

// Plain GEMM: one work-group per output tile.  Work-group ids are dealt to
// the 8 XCDs round-robin; the remap gives each XCD a contiguous run of the
// logical tile order, and the logical order walks groups of kGroupM row tiles
// column by column, so an XCD's run is a compact block of output tiles (8 x 7
// at 4096 x 7168 with 256 x 256 tiles): its L2 then serves each A and B chunk
// to several concurrently running tiles.
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_of(int64_t logical, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                        int64_t& tn) {
    const int64_t group = (int64_t)kGroupM * tiles_n;
    const int64_t first_m = (logical / group) * kGroupM;
    const int64_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
    const int64_t in_group = logical % group;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

template <int BM, int BN, int WM, int WN, int BMODE, int OUT, bool ACC, int MMA>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmParams p) {
    using Cfg = GemmCfg<BM, BN, WM, WN, BMODE>;
    __shared__ __align__(1024) uint8_t lds[2 * Cfg::kStageBytes];

    const int64_t tiles = p.tiles_m * p.tiles_n;
    const int64_t bid = blockIdx.x;
    const int64_t per_xcd = (tiles + 7) / 8;
    const int64_t xcd = bid % 8, local = bid / 8;
    const int64_t logical = xcd * per_xcd + local;
    if (logical >= tiles) return;
    int64_t tm, tn;
    tile_of(logical, p.tiles_m, p.tiles_n, tm, tn);
    TileCoord tc;
    tc.m0 = tm * BM;
    tc.n0 = tn * BN;
    tc.m_end = p.M;
    tc.group = 0;
    gemm_tile<BM, BN, WM, WN, BMODE, OUT, ACC, MMA>(p, tc, p.b, p.sb, lds);
}

// Split-K GEMM: work-group (tile, slice) runs chunks [slice * kb_split, ...)
// of one 256x256 output tile and writes the slice's FP32 partial tile to the
// workspace; splitk_reduce_kernel adds the slices in order.  For shapes whose
// tiles alone leave most CUs idle (1024 x 1024 x 65536: 16 tiles on 256
// CUs).  Slice-major order: the tiles of one slice read the same K range of
// A and B, so an XCD's run shares its L2 between them.
template <int BM, int BN, int WM, int WN, int BMODE, int MMA>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_splitk_kernel(GemmParams p) {
    using Cfg = GemmCfg<BM, BN, WM, WN, BMODE>;
    __shared__ __align__(1024) uint8_t lds[2 * Cfg::kStageBytes];

    const int64_t tiles = p.tiles_m * p.tiles_n;
    const int64_t work = tiles * p.splits;
    const int64_t bid = blockIdx.x;
    const int64_t per_xcd = (work + 7) / 8;
    const int64_t logical = (bid % 8) * per_xcd + bid / 8;
    if (logical >= work) return;
    const int64_t slice = logical / tiles;
    int64_t tm, tn;
    tile_of(logical % tiles, p.tiles_m, p.tiles_n, tm, tn);
    TileCoord tc;
    tc.m0 = tm * BM;
    tc.n0 = tn * BN;
    tc.m_end = p.M;
    tc.group = 0;
    const int64_t nk = p.K / 128;
    const int64_t kb0 = slice * p.kb_split;
    const int64_t kb1 = kb0 + p.kb_split < nk ? kb0 + p.kb_split : nk;
    gemm_tile<BM, BN, WM, WN, BMODE, kDtypeF32, false, MMA>(p, tc, p.b, p.sb, lds, kb0, kb1,
                                                            p.ws + slice * p.ws_stride, p.ldws);
}

// C = sum over slices s = 0 .. S-1 (in that order) of the FP32 partials, then
// the output conversion (bf16, fp32, or fp32 added to C).  Each thread owns 4
// consecutive columns of one row; the partials are read as 16-byte vectors.
template <int OUT, bool ACC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int64_t ldws,
                                                            int64_t ws_stride, int splits, int64_t M,
                                                            int64_t N, void* __restrict__ c, int64_t ldc,
                                                            int vec_store) {
    const int64_t quads = (N + 3) / 4;
    const int64_t total = M * quads;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / quads;
        const int64_t n = 4 * (i % quads);
        const float* src = ws + m * ldws + n;
        float4 acc = *reinterpret_cast<const float4*>(src);
        for (int sl = 1; sl < splits; ++sl) {
            const float4 v = *reinterpret_cast<const float4*>(src + sl * ws_stride);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const float r[4] = {acc.x, acc.y, acc.z, acc.w};
        if constexpr (OUT == kDtypeF32) {
            float* dst = static_cast<float*>(c) + m * ldc + n;
            if (vec_store && n + 4 <= N) {
                float4 o = acc;
                if constexpr (ACC) {
                    const float4 old = *reinterpret_cast<const float4*>(dst);
                    o.x = old.x + acc.x;
                    o.y = old.y + acc.y;
                    o.z = old.z + acc.z;
                    o.w = old.w + acc.w;
                }
                *reinterpret_cast<float4*>(dst) = o;
            } else {
                for (int e = 0; e < 4 && n + e < N; ++e) dst[e] = ACC ? dst[e] + r[e] : r[e];
            }
        } else {
            uint16_t* dst = static_cast<uint16_t*>(c) + m * ldc + n;
            if (vec_store && n + 4 <= N) {
                uint2 o;
                o.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
                o.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
                *reinterpret_cast<uint2*>(dst) = o;
            } else {
                for (int e = 0; e < 4 && n + e < N; ++e) dst[e] = f32_to_bf16(r[e]);
            }
        }
    }
}

// Strip GEMM: one work-group per 256 x 448 strip, computed as a 256x256 tile
// and then a 256x192 tile.  For shapes whose 256x256 tile count leaves the
// last round of work-groups partly empty (4096 x 7168: 448 tiles on 256
// CUs, a second round of 192), 448-wide strips give one equal unit of work
// per CU instead (256 strips of 1.75 tiles).  The host picks the layout.
// The second tile's waves are laid out 4 x 2 (64 x 96 wave tiles): a wave
// then issues 160 conversions per 96 MFMAs per chunk instead of 176 with
// 128 x 48 wave tiles.
constexpr int kStripN = 448;

template <int WM, int WN, int BMODE, int OUT, bool ACC, int MMA>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_strip_kernel(GemmParams p) {
    using Cfg1 = GemmCfg<256, 256, WM, WN, BMODE>;
    using Cfg2 = GemmCfg<256, kStripN - 256, 4, 2, BMODE>;
    static_assert(Cfg2::kStageBytes <= Cfg1::kStageBytes, "the second tile reuses the first one's LDS");
    __shared__ __align__(1024) uint8_t lds[2 * Cfg1::kStageBytes];

    const int64_t strips = p.tiles_m * p.tiles_n;  // tiles_n counts strips here
    const int64_t bid = blockIdx.x;
    const int64_t per_xcd = (strips + 7) / 8;
    const int64_t logical = (bid % 8) * per_xcd + bid / 8;
    if (logical >= strips) return;
    int64_t tm, ts;
    tile_of(logical, p.tiles_m, p.tiles_n, tm, ts);
    TileCoord tc;
    tc.m0 = tm * 256;
    tc.n0 = ts * kStripN;
    tc.m_end = p.M;
    tc.group = 0;
    gemm_tile<256, 256, WM, WN, BMODE, OUT, ACC, MMA>(p, tc, p.b, p.sb, lds);
    tc.n0 += 256;
    if (tc.n0 < p.N) {
        __syncthreads();  // every wave is done with the first tile's LDS stages
        static_assert(kStripN % 64 == 0 && Cfg2::TN == 96, "crossing points below assume these");
        if constexpr (BMODE == 0 && MMA == kMmaF16 && Cfg2::kSbPerJ) {
            // Strips start at multiples of 448 columns, so a 96-column wave
            // of this tile starts 0, 32, 64 or 96 columns into a 128-column
            // weight block and crosses into the next block at subtile 4, 2
            // or not at all.  Each wave runs the K loop specialised for its
            // crossing point (same copies and barriers in every variant), so
            // its promotion factors are formed once per row subtile.
            const int ncol = (int)(tc.n0 & 127) + (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % 2) * Cfg2::TN;
            const int js = (128 - (ncol & 127)) / 16;
            if (js == 2)
                gemm_tile<256, kStripN - 256, 4, 2, BMODE, OUT, ACC, MMA, 2>(p, tc, p.b, p.sb, lds);
            else if (js == 4)
                gemm_tile<256, kStripN - 256, 4, 2, BMODE, OUT, ACC, MMA, 4>(p, tc, p.b, p.sb, lds);
            else  // js = 6 or 8: inside one block
                gemm_tile<256, kStripN - 256, 4, 2, BMODE, OUT, ACC, MMA, Cfg2::NT>(p, tc, p.b, p.sb, lds);
        } else {
            gemm_tile<256, kStripN - 256, 4, 2, BMODE, OUT, ACC, MMA>(p, tc, p.b, p.sb, lds);
        }
    }
}

// Grouped GEMM: persistent work-groups walk a device-side tile list built from
// the group offsets (no host synchronization after routing).  An expert's rows
// are covered by 256-row tiles, except that its last row tile, when it holds
// at most 192, 128 or 64 rows, runs as a tile of that height (with Zipf expert
// sizes this cuts the padded rows from 24 % of the work, all tiles 256 high,
// to 6 %).  The list holds the tiles class by class in decreasing height
// (each class expert-major, then row tile, then column tile), so the final
// round of every work-group is a short one.
constexpr int kMaxGroups = 1024;
constexpr int kTileClasses = 4;  // 256-, 192-, 128- and 64-row tiles

// A value the caller knows to be the same in every lane, made visibly uniform
// to the compiler (it then stays in scalar registers; buffer descriptors built
// from it need no per-lane loop around each load).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Largest g < G with start[g] <= t (start is non-decreasing, start[G] > t).
__device__ __forceinline__ int find_group(const int32_t* start, int G, int64_t t) {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (start[mid] <= t) lo = mid; else hi = mid;
    }
    while (lo + 1 < G && start[lo + 1] <= t) ++lo;  // skip groups with no tiles here
    return __builtin_amdgcn_readfirstlane(lo);
}

// Height class of an expert's last row tile: 0 (256 rows), 1 (192), 2 (128)
// or 3 (64) for `last` = 1..256 rows in it.
__device__ __forceinline__ int last_tile_class(int64_t last) {
    return last > 192 ? 0 : last > 128 ? 1 : last > 64 ? 2 : 3;
}

template <int BM, int BN, int WM, int WN, int OUT, int MMA>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_kernel(GemmParams p) {
    using Cfg = GemmCfg<BM, BN, WM, WN, 0>;
    static_assert(BM == 256, "tile classes are 256, 192, 128 and 64 rows");
    // One LDS object: the two tile stages, then the tile tables and the
    // checked offsets.  (With the tables in a second __shared__ array the
    // compiler no longer tells the copies into one stage from the fragment
    // reads of the other, and waits for each chunk's copies before computing
    // it.)
    constexpr int kTables = 4 * kTileClasses * (kMaxGroups + 1);
    __shared__ __align__(1024) uint8_t lds[2 * Cfg::kStageBytes + kTables + 4 * (kMaxGroups + 1)];
    int32_t* start = reinterpret_cast<int32_t*>(lds + 2 * Cfg::kStageBytes);  // [class][G + 1]
    int32_t* off = start + kTileClasses * (kMaxGroups + 1);                     // [G + 1]

    const int G = p.groups;
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    if (threadIdx.x == 0) {
        // Offsets as the kernel uses them: clamped to [0, M] and made
        // non-decreasing, so a routing step that produced out-of-range or
        // decreasing offsets cannot send a tile outside A, its scales or C.
        int64_t prev = p.offsets[0];
        prev = prev < 0 ? 0 : prev > p.M ? p.M : prev;
        off[0] = (int32_t)prev;
        int64_t n[kTileClasses] = {0, 0, 0, 0};
        for (int g = 0; g < G; ++g) {
            int64_t hi = p.offsets[g + 1];
            hi = hi < prev ? prev : hi > p.M ? p.M : hi;
            off[g + 1] = (int32_t)hi;
            const int64_t cnt = hi - prev;
            prev = hi;
#pragma unroll
            for (int c = 0; c < kTileClasses; ++c) start[c * (kMaxGroups + 1) + g] = (int32_t)n[c];
            const int64_t rows_tiles = (cnt + BM - 1) / BM;
            if (rows_tiles > 0) {
                const int cl = last_tile_class(cnt - (rows_tiles - 1) * BM);
                n[0] += (rows_tiles - 1) * tiles_n;
                n[cl] += tiles_n;
            }
        }
#pragma unroll
        for (int c = 0; c < kTileClasses; ++c) start[c * (kMaxGroups + 1) + G] = (int32_t)n[c];
    }
    __syncthreads();
    int64_t first[kTileClasses + 1];  // first list index of each class
    first[0] = 0;
#pragma unroll
    for (int c = 0; c < kTileClasses; ++c) first[c + 1] = uniform64(first[c] + start[c * (kMaxGroups + 1) + G]);
    const int64_t total = first[kTileClasses];
    // Work-groups are dealt to the 8 XCDs round-robin.  Each round of gridDim
    // tiles is split into 8 contiguous runs, one per XCD, so that an XCD's L2
    // holds whole row tiles (all their column tiles run there) instead of
    // every XCD fetching every A row tile.
    const int64_t nwg = gridDim.x;
    const int64_t slot = nwg % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
    for (int64_t tile = slot; tile < total; tile += nwg) {
        const int cl = __builtin_amdgcn_readfirstlane(tile < first[1] ? 0 : tile < first[2] ? 1 : tile < first[3] ? 2 : 3);
        const int32_t* st = start + cl * (kMaxGroups + 1);
        const int64_t local = tile - first[cl];
        const int g = find_group(st, G, local);
        const int64_t in_g = local - st[g];
        const int64_t lo = off[g], hi = off[g + 1];
        TileCoord tc;
        tc.group = g;
        // full tiles: row tile in_g / tiles_n of the expert; a short tile is
        // the expert's last row tile
        tc.m0 = uniform64(lo + (cl == 0 ? (in_g / tiles_n) * BM : ((hi - lo + BM - 1) / BM - 1) * BM));
        tc.n0 = uniform64((in_g % tiles_n) * BN);
        tc.m_end = uniform64(hi);
        const uint8_t* b = p.b + g * p.b_group_stride;
        const float* sb = p.sb + g * p.sb_group_stride;
        if (cl == 0)
            gemm_tile<BM, BN, WM, WN, 0, OUT, false, MMA, -2, true>(p, tc, b, sb, lds);
        else if (cl == 1)
            gemm_tile<BM * 3 / 4, BN, WM, WN, 0, OUT, false, MMA, -2, true>(p, tc, b, sb, lds);
        else if (cl == 2)
            gemm_tile<BM / 2, BN, WM, WN, 0, OUT, false, MMA, -2, true>(p, tc, b, sb, lds);
        else
            gemm_tile<BM / 4, BN, WM, WN, 0, OUT, false, MMA, -2, true>(p, tc, b, sb, lds);
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------
namespace {

constexpr int kBM = 256, kBN = 256, kWM = 2, kWN = 4;

int cu_count();

GemmParams to_params(const GemmArgs& g) {
    GemmParams p;
    p.a = g.a; p.lda = g.lda; p.sa = g.sa; p.ldsa = g.ldsa;
    p.b = g.b; p.ldb = g.ldb; p.b_group_stride = g.b_group_stride;
    p.sb = g.sb; p.ldsb = g.ldsb; p.sb_group_stride = g.sb_group_stride;
    p.offsets = g.offsets; p.groups = g.groups;
    p.M = g.M; p.N = g.N; p.K = g.K; p.c = g.c; p.ldc = g.ldc;
    p.tiles_m = (g.M + kBM - 1) / kBM;
    p.tiles_n = (g.N + kBN - 1) / kBN;
    const int64_t el = g.c_dtype == kDtypeF32 ? 4 : 2;
    p.vec_store = (reinterpret_cast<uintptr_t>(g.c) % 16 == 0) && ((g.ldc * el) % 16 == 0);
    p.splits = 1;
    p.kb_split = g.K / 128;
    p.ws = nullptr;
    p.ldws = 0;
    p.ws_stride = 0;
    return p;
}

int cu_count() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return cus;
}

// Strips when they finish in fewer 64-column units of work per CU: a round of
// 256x256 tiles costs 4 units, a round of 256x448 strips 7.
bool use_strips(const GemmArgs& g) {
    const int64_t cus = cu_count();
    const int64_t tiles_m = (g.M + kBM - 1) / kBM;
    const int64_t t1 = tiles_m * ((g.N + kBN - 1) / kBN);
    const int64_t t2 = tiles_m * ((g.N + kStripN - 1) / kStripN);
    return ((t2 + cus - 1) / cus) * 7 < ((t1 + cus - 1) / cus) * 4;
}

template <int BMODE, int OUT, bool ACC, int MMA>
void launch_plain(const GemmArgs& g, GemmParams p, hipStream_t st) {
    if (use_strips(g)) {
        p.tiles_n = (g.N + kStripN - 1) / kStripN;
        const int64_t per_xcd = (p.tiles_m * p.tiles_n + 7) / 8;
        hipLaunchKernelGGL((gemm_strip_kernel<kWM, kWN, BMODE, OUT, ACC, MMA>), dim3((unsigned)(per_xcd * 8)),
                           dim3(64 * kWM * kWN), 0, st, p);
        return;
    }
    const int64_t tiles = p.tiles_m * p.tiles_n;
    const int64_t per_xcd = (tiles + 7) / 8;
    hipLaunchKernelGGL((gemm_kernel<kBM, kBN, kWM, kWN, BMODE, OUT, ACC, MMA>), dim3((unsigned)(per_xcd * 8)),
                       dim3(64 * kWM * kWN), 0, st, p);
}

template <int BMODE, int MMA>
void launch_split(const GemmArgs& g, const GemmParams& p, hipStream_t st) {
    const int64_t work = p.tiles_m * p.tiles_n * p.splits;
    const int64_t per_xcd = (work + 7) / 8;
    hipLaunchKernelGGL((gemm_splitk_kernel<kBM, kBN, kWM, kWN, BMODE, MMA>), dim3((unsigned)(per_xcd * 8)),
                       dim3(64 * kWM * kWN), 0, st, p);
    const int64_t quads = g.M * ((g.N + 3) / 4);
    const int64_t blocks = (quads + 255) / 256 < 4096 ? (quads + 255) / 256 : 4096;
    const uintptr_t ca = reinterpret_cast<uintptr_t>(g.c);
    const int vec = g.c_dtype == kDtypeF32 ? (ca % 16 == 0 && g.ldc % 4 == 0) : (ca % 8 == 0 && g.ldc % 4 == 0);
    if (g.c_dtype == kDtypeBF16)
        hipLaunchKernelGGL((splitk_reduce_kernel<kDtypeBF16, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                           p.ws, p.ldws, p.ws_stride, p.splits, g.M, g.N, g.c, g.ldc, vec);
    else if (g.accumulate)
        hipLaunchKernelGGL((splitk_reduce_kernel<kDtypeF32, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                           p.ws, p.ldws, p.ws_stride, p.splits, g.M, g.N, g.c, g.ldc, vec);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<kDtypeF32, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                           p.ws, p.ldws, p.ws_stride, p.splits, g.M, g.N, g.c, g.ldc, vec);
}

template <int MMA>
void launch_plain_mma(const GemmArgs& g, const GemmParams& p, hipStream_t st) {
    if (p.splits > 1) {
        if (g.bscale == 0)
            launch_split<0, MMA>(g, p, st);
        else
            launch_split<1, MMA>(g, p, st);
        return;
    }
    if (g.bscale == 0) {
        if (g.c_dtype == kDtypeBF16) launch_plain<0, kDtypeBF16, false, MMA>(g, p, st);
        else if (g.accumulate) launch_plain<0, kDtypeF32, true, MMA>(g, p, st);
        else launch_plain<0, kDtypeF32, false, MMA>(g, p, st);
    } else {
        if (g.c_dtype == kDtypeBF16) launch_plain<1, kDtypeBF16, false, MMA>(g, p, st);
        else if (g.accumulate) launch_plain<1, kDtypeF32, true, MMA>(g, p, st);
        else launch_plain<1, kDtypeF32, false, MMA>(g, p, st);
    }
}

template <int MMA>
void launch_grouped_mma(const GemmArgs& g, const GemmParams& p, int64_t grid, hipStream_t st) {
    if (g.c_dtype == kDtypeBF16)
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, kBN, kWM, kWN, kDtypeBF16, MMA>), dim3((unsigned)grid),
                           dim3(64 * kWM * kWN), 0, st, p);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, kBN, kWM, kWN, kDtypeF32, MMA>), dim3((unsigned)grid),
                           dim3(64 * kWM * kWN), 0, st, p);
}

}  // namespace

// Split K when the 256x256 tiles fill at most half of the CUs: as many
// slices as fit the CUs, each at least 4 chunks (512 K) long.
SplitPlan plan_splitk(int64_t M, int64_t N, int64_t K) {
    SplitPlan sp{1, K / 128, 0, 0};
    const int64_t cus = cu_count();
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int64_t nk = K / 128;
    if (tiles <= 0 || nk <= 0 || 2 * tiles > cus) return sp;
    int64_t s = cus / tiles;
    if (s > nk / 4) s = nk / 4;
    if (s < 2) return sp;
    sp.kb_split = (nk + s - 1) / s;
    sp.slices = (int)((nk + sp.kb_split - 1) / sp.kb_split);
    if (sp.slices < 2) return SplitPlan{1, nk, 0, 0};
    sp.ldws = (N + 3) / 4 * 4;
    sp.bytes = (int64_t)sp.slices * M * sp.ldws * 4;
    return sp;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
    GemmParams p = to_params(g);
    if (g.workspace) {
        const SplitPlan sp = plan_splitk(g.M, g.N, g.K);
        if (sp.slices > 1 && sp.bytes <= g.workspace_bytes) {
            p.splits = sp.slices;
            p.kb_split = sp.kb_split;
            p.ws = static_cast<float*>(g.workspace);
            p.ldws = sp.ldws;
            p.ws_stride = g.M * sp.ldws;
        }
    }
    switch (g.mma) {
        case kMmaFp8: launch_plain_mma<kMmaFp8>(g, p, st); break;
        case kMmaBf16Fold: launch_plain_mma<kMmaBf16Fold>(g, p, st); break;
        case kMmaFp8Scaled: launch_plain_mma<kMmaFp8Scaled>(g, p, st); break;
        default: launch_plain_mma<kMmaF16>(g, p, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t st) {
    const GemmParams p = to_params(g);
    const int cus = cu_count();
    // upper bound of the tile count without reading the offsets
    const int64_t tiles_n = (g.N + kBN - 1) / kBN;
    const int64_t bound = ((g.M + kBM - 1) / kBM + g.groups) * tiles_n;
    const int64_t grid = bound < cus ? (bound > 0 ? bound : 1) : cus;
    switch (g.mma) {
        case kMmaFp8: launch_grouped_mma<kMmaFp8>(g, p, grid, st); break;
        case kMmaBf16Fold: launch_grouped_mma<kMmaBf16Fold>(g, p, grid, st); break;
        case kMmaFp8Scaled: launch_grouped_mma<kMmaFp8Scaled>(g, p, grid, st); break;
        default: launch_grouped_mma<kMmaF16>(g, p, grid, st); break;
    }
    return hipGetLastError();
}

}  // namespace fp8q
