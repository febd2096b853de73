// Device building blocks of the gfx950 GEMM kernels and layout probes.
//
// Vocabulary follows the pages: A is M x K, B is K x N, the product tile of one
// workgroup is BM x BN, it walks K in K-tiles, and each 64-lane wavefront owns
// a block of matrix-instruction (MFMA) tiles, the wavefront analogue of the
// warp tile of the "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough
// (sections 2-3) and of section 4.2 of "Tensor Cores, CUTLASS and CuTe".
//
// The kernels run on the 16 x 16 matrix instructions.  Fragment ownership on
// gfx950 (64 lanes, l = lane id), as pinned by the single-wavefront probes (the
// gfx950 counterpart of the layout experiment, KingOfEgg sections 4-7):
//   v_mfma_f32_16x16x32_{bf16,f16}: operand X (A or B^T) lane l holds
//       X[row = l % 16][k = 8 (l / 16) + s], s = 0..7  (16 contiguous bytes)
//     accumulator register r of lane l holds D[row = 4 (l / 16) + r][col = l % 16]
//   v_mfma_i32_16x16x64_i8: the same with 16 int8 per lane, k = 16 (l / 16) + s.
//   v_mfma_f32_16x16x128_f8f6f4 (e4m3 operands): 32 bytes per lane -- a whole
//       128-byte K-tile row shared by 4 lanes; the kernels give lane l the two
//       16-byte fragments of the 16-bit instructions' two K-steps, bytes
//       16 (l / 16) .. +15 and 64 + 16 (l / 16) .. +15 of row l % 16, for A and
//       B alike, so every k of the row meets its partner (probed); the
//       accumulator layout is that of the 16-bit instructions.
// Both operands are "row of X with contiguous k", so the kernels keep operand
// tiles in LDS as rows of 128 bytes (one K-tile: 64 fp16/bf16 or 128 int8
// values, two K-steps) and read one 16-byte fragment per lane.  The 32 x 32
// instructions (also pinned by the probes) draw markedly more power per
// operation: under a sustained load the chip holds a clock about a fifth lower
// for them, which is why the kernels do not use them.
//
// The kernels issue MFMA(srcA = B-fragment, srcB = A-fragment), i.e. they
// compute D^T tile by tile: lane l then owns row m = l % 16 and the four
// consecutive columns n = 4 (l / 16) + 0..3 of each 16 x 16 tile, so the
// epilogue writes 4 contiguous output elements per tile.
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
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dt { F16 = 1, BF16 = 2, F32 = 3, I8 = 4, I32 = 5, E4M3 = 6 };

// Operand load modes of the tiled kernel.
enum Mode {
    KC16 = 0, // K contiguous, 16-byte-aligned rows, K a multiple of 16 bytes
    KCD = 1,  // K contiguous, 4-byte-aligned rows, any K: 16-byte loads, K tail masked
    MC16 = 2, // M (or N) contiguous, 16-byte-aligned rows, M (N) a multiple of 8
    MC8 = 3   // 8-bit, N contiguous (row-major B), 16-byte-aligned rows, N a multiple of 16
};

// Bytes of one element of a type code.
__host__ __device__ constexpr int dt_bytes(int t) { return (t == F32 || t == I32) ? 4 : (t == I8 || t == E4M3 ? 1 : 2); }

// ---------------------------------------------------------------------------
// MFMA wrappers: one 16 x 16 x (32 fp16/bf16 | 64 int8) step, 16-byte operands.
// ---------------------------------------------------------------------------
template <int T> struct Mfma;

template <> struct Mfma<BF16> {
    typedef f32x4 acc_t;
    static __device__ __forceinline__ acc_t step(u32x4 x, u32x4 y, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                       c, 0, 0, 0);
    }
    // In place, the accumulator in AGPRs (the four-wavefront tile): c = X Y + c,
    // and the first K-step's form c = X Y (accumulator operand 0, so no
    // register write precedes the instruction).  Written as assembly because
    // the compiler, given the builtin, renames the accumulator tuple between
    // the instructions and copies it through VGPRs.  Volatile, so that these
    // keep their order with respect to the wait that guards the accumulator
    // reads after the K loop.
    static __device__ __forceinline__ void step_a(u32x4 x, u32x4 y, acc_t &c)
    {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    }
    static __device__ __forceinline__ void step_a0(u32x4 x, u32x4 y, acc_t &c)
    {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(x), "v"(y));
    }
};
template <> struct Mfma<F16> {
    typedef f32x4 acc_t;
    static __device__ __forceinline__ acc_t step(u32x4 x, u32x4 y, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c,
                                                      0, 0, 0);
    }
    // in place, the accumulator in AGPRs (as for bf16)
    static __device__ __forceinline__ void step_a(u32x4 x, u32x4 y, acc_t &c)
    {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    }
    static __device__ __forceinline__ void step_a0(u32x4 x, u32x4 y, acc_t &c)
    {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(x), "v"(y));
    }
};
template <> struct Mfma<I8> {
    typedef i32x4 acc_t;
    static __device__ __forceinline__ acc_t step(u32x4 x, u32x4 y, acc_t c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, x), __builtin_bit_cast(i32x4, y), c, 0,
                                                     0, 0);
    }
    // in place, the accumulator in AGPRs (as for bf16)
    static __device__ __forceinline__ void step_a(u32x4 x, u32x4 y, acc_t &c)
    {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    }
    static __device__ __forceinline__ void step_a0(u32x4 x, u32x4 y, acc_t &c)
    {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(c) : "v"(x), "v"(y));
    }
};

// One 16 x 16 x 128 e4m3 step over a whole 128-byte K-tile row: operands are
// the two 16-byte fragments (K-steps 0 and 1 of the 16-bit layout) of each
// side.  Format code 0 (e4m3) for both operands; the scale operands are zero,
// which selects the unscaled instruction.
template <> struct Mfma<E4M3> {
    typedef f32x4 acc_t;
    static __device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi)
    {
        const uint32_t a0 = lo[0], a1 = lo[1], a2 = lo[2], a3 = lo[3];
        const uint32_t b0 = hi[0], b1 = hi[1], b2 = hi[2], b3 = hi[3];
        return i32x8{(int)a0, (int)a1, (int)a2, (int)a3, (int)b0, (int)b1, (int)b2, (int)b3};
    }
    static __device__ __forceinline__ acc_t step2(u32x4 x0, u32x4 x1, u32x4 y0, u32x4 y1, acc_t c)
    {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(join(x0, x1), join(y0, y1), c, 0, 0, 0, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// Buffer loads.  A buffer descriptor (base, size in bytes) lets every
// out-of-range vector read as zeros with no branch: the range check covers the
// lane offset plus the instruction's scalar offset.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Lane offset that the range check always rejects (slices are < 2^31 bytes).
constexpr uint32_t OOB = 0x80000000u;

// `base` and `bytes` must be the same in every lane: they are taken from the
// first active lane, so that the descriptor lives in scalar registers even where
// the compiler cannot prove that on its own (it would otherwise wrap every load
// in a loop over the distinct descriptors of the wavefront).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    base = (const void *)(((uint64_t)hi << 32) | lo);
    bytes = __builtin_amdgcn_readfirstlane(bytes);
    // word 3 = 0x00020000: raw (untyped) 32-bit data format, the gfx9-family setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes at base + voff + soff (voff per lane, soff uniform).
__device__ __forceinline__ u32x4 load16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// End of a K-tile: this wavefront's LDS accesses have completed, then all
// wavefronts meet.  One asm statement with a memory clobber, so that no memory
// access is moved across the barrier.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

// ---------------------------------------------------------------------------
// Fused epilogue on one output element, in fp32 ("Tensor Cores, CUTLASS and
// CuTe" sections 5 and 7): D = round_out(act(rs * cs * P + bias + C)), with
// P the fp32 accumulator or the int32 one converted to fp32, absent scales
// 1 and absent bias 0.  int32 output takes only + C (two's-complement
// wrap-around).  One routine for every kernel, with contraction off, so the
// kernels round identically.
// ---------------------------------------------------------------------------
struct EpiPtrs {
    const float *rs, *cs, *bias; // this batch slice's vectors (NULL: absent)
};

// The tanh form of GELU, 0.5 x (1 + tanh u), written as the equal x / (1 + e^(-2u))
// (the sum 1 + tanh u cancels for strongly negative u, the quotient does not),
// with e^(-2u) = 2^(-2u log2 e) on the hardware base-2 exponential and the
// quotient through the hardware reciprocal (each about 1 ulp; together a
// relative error near 1e-6, against some 35 instructions for the library
// exp and an IEEE division).  Strongly negative x: 2^(...) overflows to
// +inf, its reciprocal is 0 and the result -0, which is also the rounded
// value of the exact x / (1 + e^(-2u)) there.
__device__ __forceinline__ float gelu_tanh(float x)
{
#pragma clang fp contract(off)
    const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x); // sqrt(2/pi) (x + 0.044715 x^3)
    const float t = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);  // -2 log2(e) u
    return x * __builtin_amdgcn_rcpf(1.0f + t);
}

template <int O, class ST>
__device__ __forceinline__ typename Out<O>::t epi_one(int epi, int act, ST v, float rsv, float csv, float bv,
                                                      bool has_c, typename Out<O>::t c)
{
    if constexpr (O == I32) {
        return has_c ? (int)((uint32_t)v + (uint32_t)c) : (int)v;
    } else {
#pragma clang fp contract(off)
        float a = (float)v;
        if (epi) {
            a = a * rsv;
            a = a * csv;
            a = a + bv;
        }
        if (has_c)
            a = a + Out<O>::to_acc(c);
        if (act == 1)
            a = a > 0.0f ? a : 0.0f;
        else if (act == 2)
            a = gelu_tanh(a);
        // the fp32 result first, then its one rounding to the output type: the
        // empty statement keeps the last multiply or add from being fused with
        // the conversion (a mixed-precision multiply-add rounds once, to 16 bits)
        asm("" : "+v"(a));
        return Out<O>::from_acc(a);
    }
}

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
    int32_t d_nt;                               // 1: D's rows are whole 128-byte lines (streaming stores)
    int64_t a_bytes, b_bytes;                   // bytes spanned by one batch slice of A / B
    // fused epilogue: D = act(rs(i) * cs(j) * P + bias(j) + C(i,j)); NULL vectors are absent
    const float *rs, *cs, *bias;
    int64_t stride_rs, stride_cs, stride_bias;  // floats between batch slices
    int32_t act;                                // 0 none, 1 ReLU, 2 tanh-GELU
    int32_t epi;                                // 1 if any of rs, cs, bias is present
    uint64_t *phases;                           // phase log (diagnostics), NULL: off
};

// ---------------------------------------------------------------------------
// Phase log (diagnostics, off unless the host passes a log).  Thread 0 of each
// workgroup writes one record of 8 64-bit words with plain vector stores: the
// chip's 100 MHz constant clock (s_memrealtime) at the start, after the main
// loop, after the stream-K partial sums (= after the main loop elsewhere) and
// after the epilogue (or the partial store); the shader clock counter
// (s_memtime) at start and end; HW_ID and XCC_ID; the workgroup id and the
// K-tiles the record covers.  With a NULL log each call is one scalar branch.
// ---------------------------------------------------------------------------
enum PhaseSlot { PH_START = 0, PH_LOOP = 1, PH_FIX = 2, PH_END = 3, PH_CLK0 = 4, PH_CLK1 = 5, PH_HWID = 6, PH_WHO = 7 };

__device__ __forceinline__ void phase_begin(uint64_t *log, uint32_t rec, uint32_t ktiles)
{
    if (log != nullptr && threadIdx.x == 0) {
        uint64_t *r = log + (size_t)rec * 8;
        r[PH_START] = __builtin_amdgcn_s_memrealtime();
        r[PH_CLK0] = __builtin_amdgcn_s_memtime();
        const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID, bits 0-31
        const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20); // XCC_ID, bits 0-31
        r[PH_HWID] = hw | ((uint64_t)xcc << 32);
        r[PH_WHO] = blockIdx.x | ((uint64_t)ktiles << 32);
    }
}

__device__ __forceinline__ void phase_mark(uint64_t *log, uint32_t rec, int slot)
{
    if (log != nullptr && threadIdx.x == 0)
        log[(size_t)rec * 8 + slot] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void phase_end(uint64_t *log, uint32_t rec)
{
    if (log != nullptr && threadIdx.x == 0) {
        uint64_t *r = log + (size_t)rec * 8;
        r[PH_END] = __builtin_amdgcn_s_memrealtime();
        r[PH_CLK1] = __builtin_amdgcn_s_memtime();
    }
}

// Workspace of the stream-K kernel (dmu_streamk.hpp).
struct StreamKParams {
    uint32_t *flags;     // one per worker; zero outside a call
    uint32_t *error;     // set nonzero when a wait ran past its limit
    char *partials;      // one slot of BM x BN accumulators per worker
    uint32_t workers;    // W, the grid size
    uint32_t nk;         // K-tiles per tile
    uint32_t q, r;       // I = q W + r iterations (I = tiles x nk < 2^31)
    uint32_t spin_limit; // polls of a flag before a wait gives up
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

// Workgroup id -> a number in [0, n) such that XCD x (which receives ids
// x, x + 8, ...) gets a contiguous range, in increasing id order.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t n, uint32_t wg)
{
    constexpr uint32_t XCDS = 8;
    const uint32_t q = n / XCDS, r = n % XCDS;
    const uint32_t x = wg % XCDS, i = wg / XCDS;
    return x * q + (x < r ? x : r) + i; // bijection on [0, n)
}

// Tile number -> (batch, tile_m, tile_n): column-major groups of GROUP_M tile rows.
__device__ __forceinline__ TileCoord tile_coord(const GemmParams &p, uint32_t t)
{
    constexpr uint32_t GROUP_M = 4;
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

__device__ __forceinline__ TileCoord tile_of(const GemmParams &p, uint32_t wg)
{
    return tile_coord(p, xcd_remap(p.total_tiles, wg));
}

} // namespace dmu
