// Device building blocks of the gfx950 GEMM kernels and layout probes.
//
// Vocabulary follows the pages: A is M x K, B is K x N, the product tile of one
// workgroup is BM x BN, it walks K in K-tiles, and each 64-lane wavefront owns
// a block of matrix-instruction (MFMA) tiles, the wavefront analogue of the
// warp tile of the "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough
// (sections 2-3) and of section 4.2 of "Tensor Cores, CUTLASS and CuTe".
//
// MFMA fragment ownership on gfx950 (64 lanes, l = lane id), as pinned by the
// single-wavefront probes (the gfx950 counterpart of the layout experiment,
// KingOfEgg sections 4-7):
//   v_mfma_f32_32x32x16_{bf16,f16}: operand X (A or B^T) lane l holds
//       X[row = l % 32][k = 8 * (l / 32) + s], s = 0..7  (16 contiguous bytes)
//     accumulator register r of lane l holds
//       D[row = 8 * (r / 4) + 4 * (l / 32) + r % 4][col = l % 32]
//   v_mfma_i32_32x32x32_i8: the same with 16 int8 per lane, k = 16*(l/32)+s.
// Both operands are "row of X with contiguous k", so the kernels keep every
// tile K-contiguous in LDS, one 128-byte row per M (or N) index per K-tile
// (64 fp16/bf16 or 128 int8 values), and read one 16-byte fragment per lane
// with ds_read_b128.
//
// The kernels issue MFMA(srcA = B-fragment, srcB = A-fragment), i.e. they
// compute D^T tile by tile.  Lane l then owns, for each group g = r / 4, four
// consecutive columns n = 8g + 4(l/32) + 0..3 of row m = l % 32, so the
// epilogue writes 4 contiguous output elements per register group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dt { F16 = 1, BF16 = 2, F32 = 3, I8 = 4, I32 = 5 };

// Operand load modes of the tiled kernel.
enum Mode {
    KC16 = 0, // K contiguous, 16-byte-aligned rows, K a multiple of 16 bytes
    KCD = 1,  // K contiguous, 4-byte-aligned rows, any K: 16-byte loads, K tail masked
    MC16 = 2  // M (or N) contiguous, 16-byte-aligned rows, M (N) a multiple of 8
};

// Bytes of one element of a type code.
__host__ __device__ constexpr int dt_bytes(int t) { return (t == F32 || t == I32) ? 4 : (t == I8 ? 1 : 2); }

// ---------------------------------------------------------------------------
// LDS tile layout.  A tile of R rows (M or N indices) x 128 bytes (one K-tile)
// is stored row after row; the eight 16-byte chunks of a row are permuted by
// an XOR swizzle so that both the fragment reads (32 consecutive rows, same
// chunk) and the transposing writes (rows 8 apart, same chunk) spread over all
// eight chunk positions.  This plays the role of the chunk XOR swizzle of
// "Tensor Cores, CUTLASS and CuTe" section 3.5, re-derived for 128-byte rows
// and for the two access patterns used here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t swz_chunk(uint32_t row, uint32_t chunk)
{
    return chunk ^ ((row ^ (row >> 3)) & 7u);
}

__device__ __forceinline__ uint32_t lds_off(uint32_t row, uint32_t byte_in_row)
{
    return row * 128u + (swz_chunk(row, byte_in_row >> 4) << 4) + (byte_in_row & 15u);
}

// ---------------------------------------------------------------------------
// MFMA wrappers: one 32 x 32 x (16 fp16/bf16 | 32 int8) step, 16-byte operands.
// ---------------------------------------------------------------------------
template <int T> struct Mfma;

template <> struct Mfma<BF16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t step(u32x4 x, u32x4 y, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    }
};
template <> struct Mfma<F16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t step(u32x4 x, u32x4 y, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                      __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
    }
};
template <> struct Mfma<I8> {
    typedef i32x16 acc_t;
    static __device__ __forceinline__ acc_t step(u32x4 x, u32x4 y, acc_t c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, x),
                                                     __builtin_bit_cast(i32x4, y), c, 0, 0, 0);
    }
};

// Fragment of X rows [row0, row0+32) for K-step ks (0..3) of the K-tile held
// in the LDS tile at `tile`: lane l reads row row0 + l%32, bytes
// 32*ks + 16*(l/32) .. +15 of that row.
__device__ __forceinline__ u32x4 frag_read(const char *tile, uint32_t row0, uint32_t ks, uint32_t lane)
{
    const uint32_t row = row0 + (lane & 31u);
    return *reinterpret_cast<const u32x4 *>(tile + lds_off(row, ks * 32u + ((lane >> 5) << 4)));
}

// ---------------------------------------------------------------------------
// Output conversion (round to nearest even, subnormals kept).
// ---------------------------------------------------------------------------
template <int O> struct Out;
template <> struct Out<F32> {
    typedef float t;
    static __device__ __forceinline__ float from_acc(float v) { return v; }
    static __device__ __forceinline__ float to_acc(float v) { return v; }
};
template <> struct Out<BF16> {
    typedef __bf16 t;
    static __device__ __forceinline__ __bf16 from_acc(float v) { return static_cast<__bf16>(v); }
    static __device__ __forceinline__ float to_acc(__bf16 v) { return static_cast<float>(v); }
};
template <> struct Out<F16> {
    typedef _Float16 t;
    static __device__ __forceinline__ _Float16 from_acc(float v) { return static_cast<_Float16>(v); }
    static __device__ __forceinline__ float to_acc(_Float16 v) { return static_cast<float>(v); }
};
template <> struct Out<I32> {
    typedef int t;
    static __device__ __forceinline__ int from_acc(int v) { return v; }
    static __device__ __forceinline__ int to_acc(int v) { return v; }
};

// Parameters shared by every GEMM kernel (per-launch, passed by value).
struct GemmParams {
    const char *A;
    const char *B;
    const char *C;
    char *D;
    int64_t lda, ldb, ldc, ldd;                 // elements
    int64_t stride_a, stride_b, stride_c, stride_d; // elements
    int32_t M, N, K;
    int32_t batch;
    int32_t tiles_m, tiles_n;                   // tiles per batch slice
    uint32_t total_tiles;                       // tiles_m * tiles_n * batch
    int32_t a_kc, b_kc;                         // 1: operand is K-contiguous in memory
    int32_t d_vec4;                             // 1: 4-element vector access to C/D is legal
    int64_t a_bytes, b_bytes;                   // bytes spanned by one batch slice of A / B
};

// ---------------------------------------------------------------------------
// Workgroup -> (batch, tile_m, tile_n).
//
// Workgroups are handed to the 8 XCDs of the chip round-robin by id, and each
// XCD has its own L2.  The id is first remapped so that XCD x receives a
// contiguous range of tile numbers, and tile numbers are then laid out in
// column-major groups of GROUP_M tile rows, so that the tiles resident on one
// XCD share few A row panels and B column panels (the L2-aware tile order
// that "Tensor Cores, CUTLASS and CuTe" section 4.5 lists as a gap of the
// blockIdx-raster kernel).
// ---------------------------------------------------------------------------
struct TileCoord {
    int32_t b, tm, tn;
};

__device__ __forceinline__ TileCoord tile_of(const GemmParams &p, uint32_t wg)
{
    constexpr uint32_t XCDS = 8, GROUP_M = 4;
    const uint32_t n = p.total_tiles;
    const uint32_t q = n / XCDS, r = n % XCDS;
    const uint32_t x = wg % XCDS, i = wg / XCDS;
    const uint32_t t = x * q + (x < r ? x : r) + i; // bijection on [0, n)
    const uint32_t per_batch = (uint32_t)p.tiles_m * (uint32_t)p.tiles_n;
    TileCoord c;
    c.b = (int32_t)(t / per_batch);
    const uint32_t tt = t % per_batch;
    const uint32_t group_span = GROUP_M * (uint32_t)p.tiles_n;
    const uint32_t first_m = (tt / group_span) * GROUP_M;
    const uint32_t rows = min(GROUP_M, (uint32_t)p.tiles_m - first_m);
    const uint32_t u = tt % group_span;
    c.tm = (int32_t)(first_m + u % rows);
    c.tn = (int32_t)(u / rows);
    return c;
}

// ---------------------------------------------------------------------------
// Epilogue for one 32 x 32 MFMA tile computed as D^T (see the header comment):
// lane l owns row m = m0 + l%32 and columns n0 + 8g + 4(l/32) + 0..3, g = 0..3,
// with values acc[4g .. 4g+3].  D = convert(acc + C), masked at the M/N edges.
// ---------------------------------------------------------------------------
template <int O, class AccV>
__device__ __forceinline__ void store_tile(const GemmParams &p, const AccV &acc, int64_t m, int64_t n0,
                                           uint32_t lane, const char *Cb, char *Db)
{
    typedef typename Out<O>::t ot;
    if (m >= p.M)
        return;
    const ot *Crow = Cb ? reinterpret_cast<const ot *>(Cb) + m * p.ldc : nullptr;
    ot *Drow = reinterpret_cast<ot *>(Db) + m * p.ldd;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + 8 * g + 4 * (lane >> 5);
        if (p.d_vec4 && n + 3 < p.N) {
            typedef ot ov4 __attribute__((ext_vector_type(4)));
            ov4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                auto a = acc[4 * g + e];
                if (Crow)
                    a += Out<O>::to_acc(Crow[n + e]);
                v[e] = Out<O>::from_acc(a);
            }
            *reinterpret_cast<ov4 *>(Drow + n) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (n + e < p.N) {
                    auto a = acc[4 * g + e];
                    if (Crow)
                        a += Out<O>::to_acc(Crow[n + e]);
                    Drow[n + e] = Out<O>::from_acc(a);
                }
            }
        }
    }
}

} // namespace dmu
