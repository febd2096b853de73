// The direct-to-LDS tiled kernel (gemm_mfma_dl) for 16-byte-aligned operands.
//
// Global memory is copied straight into LDS with buffer_load_dwordx4 ... lds:
// each instruction moves 64 lanes x 16 bytes into 1 KiB of consecutive LDS,
// lane l filling 16-byte slot l.  The buffer descriptor's range check turns
// every out-of-range vector (rows past M/N, the K tail) into zeros without a
// branch, and no VGPRs are spent staging the next K-tile.  This is the gfx950
// counterpart of the asynchronous copy into shared memory that "Tensor Cores,
// CUTLASS and CuTe" builds its pipeline on (sections 4.2-4.3), with a
// double-buffered stage ring and one barrier per K-tile.
//
// LDS tile formats (both swizzled in 16-byte chunks):
//  * K-contiguous operand: R rows (M or N indices) x 128 bytes of K
//    (64 fp16/bf16 or 128 int8), read with ds_read_b128 (dmu_device.hpp).
//  * M/N-contiguous 16-bit operand: 64 rows (K indices) x R values, read with
//    ds_read_b64_tr_b16.  Within each group of 16 lanes that instruction
//    transposes the 16 addressed 4-value rows (pinned by the layout probe): if
//    lane j of the group addresses X[k0 + j/4][n0 + 4(j%4) .. +3], lane i
//    receives X[k0 .. k0+3][n0 + i].  Two such reads give one MFMA operand
//    (8 consecutive k of one column per lane), replacing the transposing
//    shared-memory load of the pages (ldmatrix .trans, layout experiment
//    section 5, walkthrough section 5.3).
#pragma once

#include "dmu_device.hpp"

#include <type_traits>

namespace dmu {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Offset that the buffer range check always rejects (slices are < 2^31 bytes).
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // word 3 = 0x00020000: raw (untyped) 32-bit data format, the gfx9-family setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// One 1 KiB direct copy: M0 holds the (wavefront-uniform) LDS destination and
// lane l's 16 bytes land at M0 + 16 l.  Written as inline assembly so that the
// compiler's wait-count pass does not treat the copy into one stage as a
// producer for reads of the other stage; completion is awaited explicitly
// (stage_barrier) before the barrier that publishes the stage.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr(lds)), "v"(voff), "s"(r)
                 : "memory");
}

// 4-byte direct copy used as an L2 prefetch: one lane per 128-byte line, the
// data land in a scratch corner of LDS that nothing reads.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr(lds)), "v"(voff), "s"(r)
                 : "memory");
}

// End of a K-tile: wait until this wavefront's copies of the next K-tile are in
// LDS (vmcnt(KEEP) leaves the KEEP most recent loads, the L2 prefetches of the
// K-tile after it, in flight: loads complete in issue order) and its LDS reads
// have returned, then meet the other wavefronts.  One asm statement with a
// memory clobber, so no memory access is moved across the barrier.
template <int KEEP> __device__ __forceinline__ void stage_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(KEEP) : "memory");
}

// Chunk swizzle of the transposed (K-row) tile: rows 0..3 of a group of four
// use chunk pairs shifted by 0, 2, 4, 6 so that one 16-lane transposed read
// (4 rows x 32 contiguous bytes) touches eight different chunks; rows k and
// k + 8 additionally land in opposite 128-byte halves.
__device__ __forceinline__ uint32_t swz_t(uint32_t k) { return ((k & 3u) << 1) ^ (((k >> 3) & 1u) << 3); }

// ---------------------------------------------------------------------------
// K-contiguous operand, R rows.  Instruction q (0 .. R/8-1) fills rows
// 8q .. 8q+7; lane l fills row 8q + l/8, physical chunk l%8, i.e. logical
// chunk (l%8) ^ swizzle(row).  Wavefront w issues q = w*(R/32) .. +R/32-1.
// ---------------------------------------------------------------------------
template <int R> struct KcDirect {
    static constexpr int NI = R / 32; // instructions per wavefront per K-tile
    uint32_t base[NI];                // byte offset of (row, logical chunk) at K-tile 0, or OOB
    uint32_t cb[NI];                  // byte of the chunk within a K-tile row

    __device__ __forceinline__ void init(int64_t ld_bytes, int64_t rows_valid, uint32_t wave, uint32_t lane)
    {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t q = wave * NI + i;
            const uint32_t row = 8 * q + lane / 8;
            const uint32_t chunk = (lane % 8) ^ ((row ^ (row >> 3)) & 7u);
            cb[i] = chunk * 16;
            base[i] = (int64_t)row < rows_valid ? (uint32_t)(row * ld_bytes + cb[i]) : OOB;
        }
    }
    // Copy K-tile kt (bytes kt*128 .. +127 of each row) into `tile`:
    // instruction i of this wavefront's NI.
    __device__ __forceinline__ void issue_one(int i, __amdgpu_buffer_rsrc_t r, char *tile, int kt, uint32_t k_bytes,
                                              uint32_t wave) const
    {
        const uint32_t kb0 = (uint32_t)kt * 128u;
        const uint32_t v = (base[i] != OOB && kb0 + cb[i] < k_bytes) ? base[i] + kb0 : OOB;
        dma16(r, tile + (wave * NI + i) * 1024, v);
    }
    // The same copy through registers: load_one fetches what instruction i
    // would copy (zeros when out of range), store_one writes it to its LDS slot.
    __device__ __forceinline__ u32x4 load_one(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t k_bytes) const
    {
        const uint32_t kb0 = (uint32_t)kt * 128u;
        const uint32_t v = (base[i] != OOB && kb0 + cb[i] < k_bytes) ? base[i] + kb0 : OOB;
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, 0, 0));
    }
    static __device__ __forceinline__ u32x4 frag(const char *tile, uint32_t row0, uint32_t ks, uint32_t lane)
    {
        return frag_read(tile, row0, ks, lane);
    }
    // L2 prefetch of K-tile kt: one line (one row's 128 bytes) per lane.
    uint32_t pf_base; // row * ld_bytes, or OOB
    __device__ __forceinline__ void pf_init(int64_t ld_bytes, int64_t rows_valid, uint32_t wave, uint32_t lane)
    {
        const uint32_t row = wave * (R / 4) + lane;
        pf_base = (lane < R / 4 && (int64_t)row < rows_valid) ? (uint32_t)(row * ld_bytes) : OOB;
    }
    __device__ __forceinline__ void prefetch(__amdgpu_buffer_rsrc_t r, char *junk, int kt, uint32_t k_bytes) const
    {
        const uint32_t kb0 = (uint32_t)kt * 128u;
        dma4(r, junk, (pf_base != OOB && kb0 < k_bytes) ? pf_base + kb0 : OOB);
    }
};

// ---------------------------------------------------------------------------
// M/N-contiguous 16-bit operand: 64 K-rows x R values (2R bytes per row).
// Instruction q fills rows q*RPI .. +RPI-1 (RPI = 512/R rows of 2R bytes);
// lane l fills row q*RPI + l/CPR, physical chunk l%CPR (CPR = R/8 chunks per
// row), i.e. logical chunk (l%CPR) ^ swz_t(row).
// ---------------------------------------------------------------------------
template <int R> struct McDirect {
    static_assert(R == 128 || R == 256, "transposed tile of 128 or 256 values");
    static constexpr int CPR = R / 8;
    static constexpr int RPI = 64 / CPR;
    static constexpr int NI = R / 32;
    uint32_t base[NI]; // (k*ld + n) bytes at K-tile 0, or OOB
    uint32_t krow[NI]; // K-row within the tile

    __device__ __forceinline__ void init(int64_t ld_bytes, int64_t mn_valid, uint32_t wave, uint32_t lane)
    {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t q = wave * NI + i;
            const uint32_t k = q * RPI + lane / CPR;
            const uint32_t chunk = (lane % CPR) ^ swz_t(k);
            krow[i] = k;
            base[i] = (int64_t)(8 * chunk) < mn_valid ? (uint32_t)(k * ld_bytes + chunk * 16) : OOB;
        }
    }
    // Instruction i of this wavefront's NI copies of K-tile kt;
    // ld_bytes_tile = 64 * ld_bytes is the byte step between K-tiles.
    __device__ __forceinline__ void issue_one(int i, __amdgpu_buffer_rsrc_t r, char *tile, int kt, uint32_t k_rows,
                                              uint32_t ld_bytes_tile, uint32_t wave) const
    {
        const uint32_t k0 = (uint32_t)kt * 64u;
        const uint32_t v = (base[i] != OOB && k0 + krow[i] < k_rows) ? base[i] + (uint32_t)kt * ld_bytes_tile : OOB;
        dma16(r, tile + (wave * NI + i) * 1024, v);
    }
    __device__ __forceinline__ u32x4 load_one(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t k_rows,
                                              uint32_t ld_bytes_tile) const
    {
        const uint32_t k0 = (uint32_t)kt * 64u;
        const uint32_t v = (base[i] != OOB && k0 + krow[i] < k_rows) ? base[i] + (uint32_t)kt * ld_bytes_tile : OOB;
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, 0, 0));
    }
    // Operand fragment of columns [c0, c0+32) at K-step ks: lane l gets column
    // c0 + l%32, k = 16ks + 8(l/32) + 0..7.
    static __device__ __forceinline__ u32x4 frag(const char *tile, uint32_t c0, uint32_t ks, uint32_t lane)
    {
        const uint32_t g = lane >> 4, j = lane & 15u;
        const uint32_t n = c0 + 16 * (g & 1u) + 4 * (j & 3u);
        const uint32_t chunk = n >> 3, inner = (n & 7u) * 2;
        const uint32_t k = 16 * ks + 8 * (g >> 1) + (j >> 2);
        const uint32_t a0 = k * (2 * R) + ((chunk ^ swz_t(k)) << 4) + inner;
        const uint32_t a1 = (k + 4) * (2 * R) + ((chunk ^ swz_t(k + 4)) << 4) + inner;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(tile + a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(tile + a1));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
    // L2 prefetch of K-tile kt: the tile is 64 K-rows of 2R bytes = R lines of
    // 128 bytes; lane l of wavefront w takes line w*R/4 + l.
    uint32_t pf_base; // k * ld_bytes + part * 128, or OOB
    uint32_t pf_k;
    __device__ __forceinline__ void pf_init(int64_t ld_bytes, int64_t mn_valid, uint32_t wave, uint32_t lane)
    {
        constexpr uint32_t LPR = 2 * R / 128; // lines per K-row
        const uint32_t line = wave * (R / 4) + lane;
        pf_k = line / LPR;
        const uint32_t part = line % LPR;
        pf_base = (lane < R / 4 && (int64_t)(part * 64) < mn_valid) ? (uint32_t)(pf_k * ld_bytes + part * 128) : OOB;
    }
    __device__ __forceinline__ void prefetch(__amdgpu_buffer_rsrc_t r, char *junk, int kt, uint32_t k_rows,
                                             uint32_t ld_bytes_tile) const
    {
        const uint32_t k0 = (uint32_t)kt * 64u;
        dma4(r, junk, (pf_base != OOB && k0 + pf_k < k_rows) ? pf_base + (uint32_t)kt * ld_bytes_tile : OOB);
    }
};

// ---------------------------------------------------------------------------
// Epilogue through LDS.  A wavefront owns (32 MT) x (32 NT) results; lane l
// holds, per 32 x 32 MFMA tile and register group g, four consecutive columns
// of one row (the D^T orientation, dmu_device.hpp).  Written straight to
// memory that is 32 rows x 16 bytes per store instruction; here each 32-row
// stripe is first parked in the wavefront's own LDS area as fp32, then read
// back row-contiguous so that each store instruction writes two full rows of
// 32 NT values (whole cache lines), with C added and the result converted on
// the way out (the shared-memory route to wide stores that the walkthrough's
// section 7.5 and "Tensor Cores, CUTLASS and CuTe" section 4.5 point to).
// ---------------------------------------------------------------------------
template <int O, int MT, int NT, class AccT>
__device__ __forceinline__ void store_staged(const GemmParams &p, const AccT (&acc)[MT][NT], char *lds,
                                             int64_t m_base, int64_t n_base, uint32_t lane, const char *Cb, char *Db)
{
    typedef typename Out<O>::t ot;
    typedef decltype(acc[0][0][0]) sref;
    typedef typename std::remove_const<typename std::remove_reference<sref>::type>::type st; // float or int
    typedef st st4 __attribute__((ext_vector_type(4)));
    constexpr int COLS = 32 * NT;
    constexpr int PITCH = COLS * 4 + 16; // bytes per parked row (+16 spreads rows over the banks)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
        // park: lane l writes 4 values of row l%32 per (ni, g)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t col = ni * 32 + 8 * g + 4 * (lane >> 5);
                st4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = acc[mi][ni][4 * g + e];
                *reinterpret_cast<st4 *>(lds + (lane & 31u) * PITCH + col * 4) = v;
            }
        // read back row-contiguous: lanes 0..31 and 32..63 take two rows
        constexpr int LPR = COLS / 4; // lanes per row
#pragma unroll 4
        for (int it = 0; it < 32 * LPR / 64; ++it) {
            const uint32_t idx = it * 64 + lane;
            const uint32_t row = idx / LPR, col = (idx % LPR) * 4;
            const st4 v = *reinterpret_cast<const st4 *>(lds + row * PITCH + col * 4);
            const int64_t m = m_base + mi * 32 + row, n = n_base + col;
            if (m >= p.M)
                continue;
            const ot *Crow = Cb ? reinterpret_cast<const ot *>(Cb) + m * p.ldc : nullptr;
            ot *Drow = reinterpret_cast<ot *>(Db) + m * p.ldd;
            if (p.d_vec4 && n + 3 < p.N) {
                typedef ot ov4 __attribute__((ext_vector_type(4)));
                ov4 o;
                if (Crow) {
                    const ov4 c = *reinterpret_cast<const ov4 *>(Crow + n);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        st a = v[e];
                        a += Out<O>::to_acc(c[e]);
                        o[e] = Out<O>::from_acc(a);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        st a = v[e];
                        o[e] = Out<O>::from_acc(a);
                    }
                }
                *reinterpret_cast<ov4 *>(Drow + n) = o;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e < p.N) {
                        st a = v[e];
                        if (Crow)
                            a += Out<O>::to_acc(Crow[n + e]);
                        Drow[n + e] = Out<O>::from_acc(a);
                    }
                }
            }
        }
    }
}

template <int MODE, int R> struct DirectOf;
template <int R> struct DirectOf<KC16, R> { typedef KcDirect<R> type; };
template <int R> struct DirectOf<MC16, R> { typedef McDirect<R> type; };

template <int T, int O, int BM, int BN, int AMODE, int BMODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_mfma_dl(GemmParams p)
{
    constexpr int E = T == I8 ? 1 : 2;
    constexpr int WTM = BM / 2, WTN = BN / 2; // 2 x 2 wavefronts
    constexpr int MT = WTM / 32, NT = WTN / 32;
    constexpr int ABYTES = BM * 128, STAGE = (BM + BN) * 128;
    typedef typename Mfma<T>::acc_t acc_t;
    typedef typename DirectOf<AMODE, BM>::type ATile;
    typedef typename DirectOf<BMODE, BN>::type BTile;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + 1024];
    char *const junk = smem + 2 * STAGE; // landing area of the L2 prefetches (never read)

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    const TileCoord tc = tile_of(p, blockIdx.x);
    const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;

    // Buffer descriptors cover this tile's part of each operand, from its first
    // row (K-contiguous) or column (M/N-contiguous) to the end of the batch slice.
    const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
    const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;
    const int64_t a_start = AMODE == KC16 ? m0 * p.lda * E : m0 * E;
    const int64_t b_start = BMODE == KC16 ? n0 * p.ldb * E : n0 * E;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_start, (uint32_t)(p.a_bytes - a_start));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_start, (uint32_t)(p.b_bytes - b_start));

    ATile ta;
    BTile tb;
    ta.init(p.lda * E, p.M - m0, wave, lane);
    tb.init(p.ldb * E, p.N - n0, wave, lane);
    ta.pf_init(p.lda * E, p.M - m0, wave, lane);
    tb.pf_init(p.ldb * E, p.N - n0, wave, lane);
    const uint32_t k_bytes = (uint32_t)p.K * E;
    const uint32_t a_tile_step = (uint32_t)(64 * p.lda * E), b_tile_step = (uint32_t)(64 * p.ldb * E);

    acc_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = acc_t{};

    const int nk = (int)(((int64_t)p.K * E + 127) / 128);

    // The copy work of one K-tile as single 16-byte-per-lane transfers: the A
    // tile's NA, then the B tile's NB.  Transfer c fills 1 KiB of the stage,
    // lane l writing bytes 16 l .. 16 l + 15 of it.
    constexpr int NA = ATile::NI, NB = BTile::NI, NLD = NA + NB;
    auto load_one = [&](int c, int kt) -> u32x4 {
        if (c < NA) {
            if constexpr (AMODE == KC16)
                return ta.load_one(c, ra, kt, k_bytes);
            else
                return ta.load_one(c, ra, kt, (uint32_t)p.K, a_tile_step);
        } else {
            if constexpr (BMODE == KC16)
                return tb.load_one(c - NA, rb, kt, k_bytes);
            else
                return tb.load_one(c - NA, rb, kt, (uint32_t)p.K, b_tile_step);
        }
    };
    auto store_one = [&](int c, char *stage, const u32x4 &v) {
        char *dst = c < NA ? stage + (wave * NA + c) * 1024 : stage + ABYTES + (wave * NB + (c - NA)) * 1024;
        *reinterpret_cast<u32x4 *>(dst + lane * 16) = v;
    };
    // Fragment f (0..MT-1: A rows; MT..MT+NT-1: B columns) of K-step ks.
    auto read_one = [&](int f, const char *stage, int ks, u32x4 *af, u32x4 *bf) {
        if (f < MT)
            af[f] = ATile::frag(stage, wm * WTM + f * 32, ks, lane);
        else
            bf[f - MT] = BTile::frag(stage + ABYTES, wn * WTN + (f - MT) * 32, ks, lane);
    };

    // Fragment registers: a double buffer over the K-steps, carried across
    // K-tiles (K-step 0 of the next K-tile is read while the last MFMAs of the
    // current one run).  stg holds the next K-tile between its global loads
    // and its LDS writes.
    u32x4 af[2][MT], bfr[2][NT], stg[NLD];

    if (nk > 0) {
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            stg[c] = load_one(c, 0);
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            store_one(c, smem, stg[c]);
        stage_barrier<0>();
#pragma unroll
        for (int f = 0; f < MT + NT; ++f)
            read_one(f, smem, 0, af[0], bfr[0]);
    }

    // The K-tile body is an explicit issue schedule (a scheduling barrier after
    // every slot).  MFMA q of a K-step is followed by the read of its share of
    // the next K-step's fragments; the global loads of the next K-tile ride on
    // the MFMAs of K-steps 0 and 1, its LDS writes on those of K-steps 2 and 3,
    // so the matrix cores never wait behind a burst of memory instructions.
    // After the last K-tile the same schedule runs on "K-tile nk", which lies
    // wholly past K: the buffer range check turns its loads into zeros, so the
    // body needs no branches (branches around the loads make the compiler
    // drain the memory counters at every join).
    constexpr int MN = MT * NT, NF = MT + NT;
    for (int kt = 0; kt < nk; ++kt) {
        const char *cur = smem + (kt & 1) * STAGE;
        char *nxt = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
            const int c = ks & 1, n = c ^ 1;
#pragma unroll
            for (int q = 0; q < MN; ++q) {
                acc[q / NT][q % NT] = Mfma<T>::step(bfr[c][q % NT], af[c][q / NT], acc[q / NT][q % NT]);
#pragma unroll
                for (int f = q * NF / MN; f < (q + 1) * NF / MN; ++f)
                    read_one(f, cur, ks + 1, af[n], bfr[n]);
                if (ks < 2) { // global loads [slot*NLD/(2 MN), (slot+1)*NLD/(2 MN)) of K-tile kt+1
                    const int slot = ks * MN + q;
#pragma unroll
                    for (int ci = slot * NLD / (2 * MN); ci < (slot + 1) * NLD / (2 * MN); ++ci)
                        stg[ci] = load_one(ci, kt + 1);
                } else { // LDS writes, first two thirds
#pragma unroll
                    for (int ci = q * NLD / (3 * MN / 2); ci < (q + 1) * NLD / (3 * MN / 2); ++ci)
                        store_one(ci, nxt, stg[ci]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // K-step 3: half of its MFMAs with the remaining LDS writes, the stage
        // hand-over, then the other half with the first reads of K-tile kt+1.
#pragma unroll
        for (int q = 0; q < MN / 2; ++q) {
            acc[q / NT][q % NT] = Mfma<T>::step(bfr[1][q % NT], af[1][q / NT], acc[q / NT][q % NT]);
            const int slot = MN + q;
#pragma unroll
            for (int ci = slot * NLD / (3 * MN / 2); ci < (slot + 1) * NLD / (3 * MN / 2); ++ci)
                store_one(ci, nxt, stg[ci]);
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_barrier<0>();
#pragma unroll
        for (int q = MN / 2; q < MN; ++q) {
            acc[q / NT][q % NT] = Mfma<T>::step(bfr[1][q % NT], af[1][q / NT], acc[q / NT][q % NT]);
            const int h = q - MN / 2; // fragments [h*NF/(MN/2), (h+1)*NF/(MN/2)) of K-step 0, K-tile kt+1
#pragma unroll
            for (int f = h * NF / (MN / 2); f < (h + 1) * NF / (MN / 2); ++f)
                read_one(f, nxt, 0, af[0], bfr[0]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    const char *Cb = p.C ? p.C + (int64_t)tc.b * p.stride_c * dt_bytes(O) : nullptr;
    char *Db = p.D + (int64_t)tc.b * p.stride_d * dt_bytes(O);
    // Every wavefront is past the last barrier, so no one reads the stages any
    // more: each wavefront parks its results in its own part of them.
    constexpr int PARK = 32 * (32 * NT * 4 + 16);
    static_assert(4 * PARK <= 2 * STAGE, "parking area fits in the stages");
    store_staged<O, MT, NT>(p, acc, smem + wave * PARK, m0 + wm * WTM, n0 + wn * WTN, lane, Cb, Db);
}

} // namespace dmu
