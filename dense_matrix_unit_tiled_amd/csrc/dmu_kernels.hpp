// GEMM kernels for gfx950: D = A*B + C on the MFMA matrix cores.
//
// Two kernel families share the fragment layout, the LDS tile format, the
// tile order and the epilogue of dmu_device.hpp:
//
//  gemm_mfma   the tiled kernel.  A workgroup of 256 threads (4 wavefronts of
//              64 lanes, arranged WGM x WGN) computes a BM x BN tile; each
//              wavefront owns a (BM/WGM) x (BN/WGN) block of 32 x 32 MFMA
//              tiles.  K is walked in K-tiles of 128 bytes per row (64
//              fp16/bf16 or 128 int8 values).  Global memory is read with
//              coalesced 16-byte (or 4-byte) vector loads into registers while
//              the MFMAs consume the previous K-tile from LDS; the registers
//              are then written into the other half of a double-buffered LDS
//              ring, with one barrier per K-tile.  Out-of-range rows and the K
//              tail are zero-filled; the epilogue masks the M/N edges.
//              Three-level tiling (workgroup -> wavefront -> instruction) as in
//              the "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough
//              (sections 2-6) and "Tensor Cores, CUTLASS and CuTe" section 4.2,
//              re-sized for 64-lane wavefronts and 32 x 32 instructions; the
//              double-buffered stage ring replaces that page's three-stage
//              cp.async pipeline (section 4.3).
//
//  gemm_generic  a plain fallback for operands whose alignment rules out
//              vector loads: 64 x 64 tiles, element-by-element loads, one LDS
//              buffer with two barriers per K-tile (the simplest correct form,
//              as in the walkthrough's kernel).  It issues exactly the same
//              MFMA sequence per output element as gemm_mfma, so the two are
//              bit-identical on the same inputs.
#pragma once

#include "dmu_device.hpp"

#include <type_traits>

namespace dmu {

template <int T> struct In;
template <> struct In<F16> { static constexpr int bytes = 2; };
template <> struct In<BF16> { static constexpr int bytes = 2; };
template <> struct In<I8> { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// K-contiguous operand: an R x 128-byte K-tile, rows = M (or N) indices.
// Thread t loads vectors t, t+256, ...; eight (or 32) consecutive threads read
// one 128-byte row segment, so every wavefront load is fully coalesced.
// ---------------------------------------------------------------------------
template <int R, int VB> struct KcTile {
    static constexpr int VPR = 128 / VB;
    static constexpr int NV = R * VPR / 256;
    static_assert(NV * 256 == R * VPR, "tile rows must fill the workgroup");
    typedef typename std::conditional<VB == 16, u32x4, uint32_t>::type vec_t;
    vec_t v[NV];

    // base: this batch slice; ld_bytes: leading dimension in bytes;
    // row0/rows_valid: first row of the tile and rows left in the matrix;
    // kb0/kb_valid: first byte of the K-tile in a row and bytes left in the row.
    __device__ __forceinline__ void load(const char *base, int64_t ld_bytes, int64_t row0, int64_t rows_valid,
                                         int64_t kb0, int64_t kb_valid, uint32_t tid)
    {
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const uint32_t idx = tid + 256u * q;
            const uint32_t row = idx / VPR, cb = (idx % VPR) * VB;
            if ((int64_t)row < rows_valid && (int64_t)cb < kb_valid)
                v[q] = *reinterpret_cast<const vec_t *>(base + (row0 + row) * ld_bytes + kb0 + cb);
            else
                v[q] = vec_t{};
        }
    }
    __device__ __forceinline__ void store(char *tile, uint32_t tid) const
    {
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const uint32_t idx = tid + 256u * q;
            const uint32_t row = idx / VPR, cb = (idx % VPR) * VB;
            *reinterpret_cast<vec_t *>(tile + lds_off(row, cb)) = v[q];
        }
    }
};

// ---------------------------------------------------------------------------
// M/N-contiguous 16-bit operand (row-major B, column-major A): memory rows are
// K indices.  Thread t < R owns an 8 (k) x 8 (m/n) block: eight 16-byte loads
// (rows k..k+7), an in-register 8 x 8 transpose of 16-bit values, and eight
// 16-byte LDS writes, one per m/n row, each holding 8 consecutive k.  This
// replaces the transposing shared-memory read of the pages (ldmatrix .trans,
// layout experiment section 5; walkthrough section 5.3) with a transpose on
// the way into LDS, so that every fragment read stays a plain ds_read_b128.
// ---------------------------------------------------------------------------
template <int R> struct McTile {
    static_assert(R <= 256 && R % 8 == 0, "one 8x8 block per thread");
    static constexpr int GROUPS = R / 8; // 8-wide m/n groups per tile
    u32x4 v[8];

    // base: this batch slice; ld_bytes: bytes between consecutive k rows;
    // mn0/mn_valid: first m/n of the tile and m/n left (a multiple of 8);
    // k0/k_valid: first k of the K-tile and k rows left.
    __device__ __forceinline__ void load(const char *base, int64_t ld_bytes, int64_t mn0, int64_t mn_valid,
                                         int64_t k0, int64_t k_valid, uint32_t tid)
    {
        if (tid >= (uint32_t)R)
            return;
        const uint32_t kg = tid / GROUPS, mg = tid % GROUPS;
        const bool mn_ok = (int64_t)(8 * mg) < mn_valid;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t k = 8 * kg + r;
            if (mn_ok && k < k_valid)
                v[r] = *reinterpret_cast<const u32x4 *>(base + (k0 + k) * ld_bytes + (mn0 + 8 * mg) * 2);
            else
                v[r] = u32x4{};
        }
    }
    __device__ __forceinline__ void store(char *tile, uint32_t tid) const
    {
        if (tid >= (uint32_t)R)
            return;
        const uint32_t kg = tid / GROUPS, mg = tid % GROUPS;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 o;
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const uint32_t lo = v[2 * pr][c >> 1], hi = v[2 * pr + 1][c >> 1];
                o[pr] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<u32x4 *>(tile + lds_off(8 * mg + c, 16 * kg)) = o;
        }
    }
};

template <int MODE, int R> struct TileOf;
template <int R> struct TileOf<KC16, R> { typedef KcTile<R, 16> type; };
template <int R> struct TileOf<KC4, R> { typedef KcTile<R, 4> type; };
template <int R> struct TileOf<MC16, R> { typedef McTile<R> type; };

// Load K-tile kt of one operand into registers.  For K-contiguous operands the
// matrix rows are the tile rows; for M/N-contiguous ones they are K indices.
template <int MODE, int T, class Tile>
__device__ __forceinline__ void load_operand(Tile &t, const char *base, int64_t ld, int64_t mn0, int64_t mn,
                                             int64_t K, int kt, uint32_t tid)
{
    constexpr int E = In<T>::bytes;
    if (MODE == MC16)
        t.load(base, ld * E, mn0, mn - mn0, (int64_t)kt * (128 / E), K - (int64_t)kt * (128 / E), tid);
    else
        t.load(base, ld * E, mn0, mn - mn0, (int64_t)kt * 128, K * E - (int64_t)kt * 128, tid);
}

template <int T, int O, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_mfma(GemmParams p)
{
    constexpr int E = In<T>::bytes;
    constexpr int WTM = BM / WGM, WTN = BN / WGN; // wavefront tile
    constexpr int MT = WTM / 32, NT = WTN / 32;   // MFMA tiles per wavefront
    constexpr int STAGE = (BM + BN) * 128;
    static_assert(WGM * WGN == 4, "four wavefronts");
    typedef typename Mfma<T>::acc_t acc_t;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t wm = wave / WGN, wn = wave % WGN;
    const TileCoord tc = tile_of(p, blockIdx.x);
    const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
    const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
    const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;

    acc_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = acc_t{};

    typename TileOf<AMODE, BM>::type ta;
    typename TileOf<BMODE, BN>::type tb;
    const int nk = (int)(((int64_t)p.K * E + 127) / 128);

    if (nk > 0) {
        load_operand<AMODE, T>(ta, Ab, p.lda, m0, p.M, p.K, 0, tid);
        load_operand<BMODE, T>(tb, Bb, p.ldb, n0, p.N, p.K, 0, tid);
        ta.store(smem, tid);
        tb.store(smem + BM * 128, tid);
        __syncthreads();
    }

    for (int kt = 0; kt < nk; ++kt) {
        const char *As = smem + (kt & 1) * STAGE;
        const char *Bs = As + BM * 128;
        const bool more = kt + 1 < nk;
        if (more) { // next K-tile: global -> registers, in flight during the MFMAs
            load_operand<AMODE, T>(ta, Ab, p.lda, m0, p.M, p.K, kt + 1, tid);
            load_operand<BMODE, T>(tb, Bb, p.ldb, n0, p.N, p.K, kt + 1, tid);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 af[MT], bfr[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                af[i] = frag_read(As, wm * WTM + i * 32, ks, lane);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bfr[j] = frag_read(Bs, wn * WTN + j * 32, ks, lane);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = Mfma<T>::step(bfr[j], af[i], acc[i][j]);
        }
        if (more) { // registers -> the other LDS stage (last read one K-tile ago)
            char *nxt = smem + ((kt + 1) & 1) * STAGE;
            ta.store(nxt, tid);
            tb.store(nxt + BM * 128, tid);
        }
        __syncthreads();
    }

    const char *Cb = p.C ? p.C + (int64_t)tc.b * p.stride_c * dt_bytes(O) : nullptr;
    char *Db = p.D + (int64_t)tc.b * p.stride_d * dt_bytes(O);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            store_tile<O>(p, acc[i][j], m0 + wm * WTM + i * 32 + (lane & 31u), n0 + wn * WTN + j * 32, lane,
                          Cb, Db);
}

// ---------------------------------------------------------------------------
// Fallback: any alignment, any layout.  64 x 64 tile, wavefront w owns the
// 32 x 32 MFMA tile (w / 2, w % 2).
// ---------------------------------------------------------------------------
template <int T, int E> struct Elem;
template <int T> struct Elem<T, 2> { typedef uint16_t t; };
template <int T> struct Elem<T, 1> { typedef uint8_t t; };

template <int T>
__device__ __forceinline__ void generic_fill(char *tile, const char *base, int64_t ld, bool kc, int64_t mn0,
                                             int64_t MN, int64_t k0, int64_t K, uint32_t tid)
{
    constexpr int E = In<T>::bytes;
    constexpr int EPR = 128 / E; // elements per LDS row (one K-tile)
    typedef typename Elem<T, E>::t et;
    const et *src = reinterpret_cast<const et *>(base);
#pragma unroll 4
    for (int q = 0; q < 64 * EPR / 256; ++q) {
        const uint32_t idx = tid + 256u * q;
        // consecutive threads walk the memory-contiguous dimension
        const uint32_t row = kc ? idx / EPR : idx % 64u;
        const uint32_t ke = kc ? idx % EPR : idx / 64u;
        const int64_t mn = mn0 + row, k = k0 + ke;
        et v = 0;
        if (mn < MN && k < K)
            v = src[kc ? mn * ld + k : mn + k * ld];
        *reinterpret_cast<et *>(tile + lds_off(row, ke * E)) = v;
    }
}

template <int T, int O>
__global__ void __launch_bounds__(256) gemm_generic(GemmParams p)
{
    constexpr int E = In<T>::bytes;
    typedef typename Mfma<T>::acc_t acc_t;
    __shared__ __attribute__((aligned(1024))) char smem[128 * 128];

    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    const TileCoord tc = tile_of(p, blockIdx.x);
    const int64_t m0 = (int64_t)tc.tm * 64, n0 = (int64_t)tc.tn * 64;
    const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
    const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;
    acc_t acc = acc_t{};
    const int nk = (int)(((int64_t)p.K * E + 127) / 128);
    for (int kt = 0; kt < nk; ++kt) {
        const int64_t k0 = (int64_t)kt * (128 / E);
        generic_fill<T>(smem, Ab, p.lda, p.a_kc != 0, m0, p.M, k0, p.K, tid);
        generic_fill<T>(smem + 64 * 128, Bb, p.ldb, p.b_kc != 0, n0, p.N, k0, p.K, tid);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 af = frag_read(smem, wm * 32, ks, lane);
            const u32x4 bfr = frag_read(smem + 64 * 128, wn * 32, ks, lane);
            acc = Mfma<T>::step(bfr, af, acc);
        }
        __syncthreads();
    }
    const char *Cb = p.C ? p.C + (int64_t)tc.b * p.stride_c * dt_bytes(O) : nullptr;
    char *Db = p.D + (int64_t)tc.b * p.stride_d * dt_bytes(O);
    store_tile<O>(p, acc, m0 + wm * 32 + (lane & 31u), n0 + wn * 32, lane, Cb, Db);
}

} // namespace dmu
