// The tiled kernel (gemm_tiled) for operands whose rows are at least 4-byte
// aligned (K-contiguous) or 16-byte aligned (M/N-contiguous).
//
// A workgroup of 64*WGM*WGN threads (WGM x WGN wavefronts) computes a BM x BN
// tile of D; each wavefront owns a (BM/WGM) x (BN/WGN) block of 32 x 32 MFMA
// tiles.  K is walked in K-tiles of 128 bytes per row (64 fp16/bf16 or 128
// int8 values), each split into 4 MFMA K-steps.  Three-level tiling
// (workgroup, wavefront, instruction) as in the
// "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough (sections 2-6) and
// "Tensor Cores, CUTLASS and CuTe" section 4.2, re-sized for 64-lane
// wavefronts, 32 x 32 instructions, 160 KiB of LDS, and -- with 8 wavefronts
// -- two wavefronts per SIMD, so that one covers the other's memory waits.
//
// Data path of one K-tile:
//   global -> VGPR   buffer_load_dwordx4 through a buffer descriptor: every
//                    out-of-range vector (rows past M/N, the K tail, the
//                    K-tile after the last) reads as zeros without a branch.
//   VGPR -> LDS      ds_write_b128 into the other half of a double-buffered
//                    stage ring; each load/write pair moves 1 KiB, lane l
//                    handling bytes 16 l .. 16 l + 15 of it.
//   LDS -> VGPR      MFMA operand fragments.  A K-contiguous operand is kept
//                    as R rows x 128 bytes and read with one ds_read_b128 per
//                    fragment (dmu_device.hpp).  An M/N-contiguous 16-bit
//                    operand (row-major B, column-major A) is kept as it lies
//                    in memory, 64 K-rows x R values, and read with two
//                    ds_read_b64_tr_b16 per fragment: within each group of 16
//                    lanes that instruction transposes the 16 addressed
//                    4-value rows (pinned by the layout probe), so if lane j
//                    of the group addresses X[k0 + j/4][n0 + 4(j%4) .. +3],
//                    lane i receives X[k0 .. k0+3][n0 + i].  This replaces the
//                    transposing shared-memory load of the pages (ldmatrix
//                    .trans, layout experiment section 5; walkthrough 5.3).
// Both LDS formats are XOR-swizzled in 16-byte chunks.  One barrier per
// K-tile hands a stage over (the stage ring of "Tensor Cores, CUTLASS and
// CuTe" section 4.3, two stages deep here).
//
// The K-tile body is an explicit issue schedule: every MFMA is followed by a
// few of the memory instructions the wavefront owes (next K-step's fragment
// reads; in K-steps 0-2 the LDS writes of the next K-tile, each followed by the
// global load of the K-tile after it into the same staging registers), with
// scheduling barriers so that the compiler keeps that order and the matrix
// core never waits behind a burst of memory instructions.
#pragma once

#include "dmu_device.hpp"

#include <type_traits>

namespace dmu {

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Offset that the buffer range check always rejects (slices are < 2^31 bytes).
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // word 3 = 0x00020000: raw (untyped) 32-bit data format, the gfx9-family setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// End of a K-tile: this wavefront's LDS accesses have completed, then all
// wavefronts meet.  One asm statement with a memory clobber, so that no memory
// access is moved across the barrier.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Chunk swizzle of the transposed (K-row) tile: rows 0..3 of a group of four
// use chunk pairs shifted by 0, 2, 4, 6 so that one 16-lane transposed read
// (4 rows x 32 contiguous bytes) touches eight different chunks; rows k and
// k + 8 additionally land in opposite 128-byte halves.
__device__ __forceinline__ uint32_t swz_t(uint32_t k) { return ((k & 3u) << 1) ^ (((k >> 3) & 1u) << 3); }

// ---------------------------------------------------------------------------
// K-contiguous operand, R rows x 128 bytes per K-tile, NW wavefronts.
// Transfer i of wavefront w (i < NL = R/(8 NW)) moves rows 8q .. 8q+7,
// q = w*NL + i: lane l fetches row 8q + l/8, logical chunk (l%8) ^
// swizzle(row), into physical chunk l%8.  Eight consecutive lanes read one
// whole 128-byte row segment.
// ---------------------------------------------------------------------------
template <int R, int NW, bool MASK> struct KcStage {
    static constexpr int NL = R / (8 * NW);
    static_assert(NL * 8 * NW == R, "whole 1 KiB transfers per wavefront");
    uint32_t base[NL]; // byte offset at K-tile 0, or OOB
    uint32_t cb[NL];   // byte of the chunk within a K-tile row

    __device__ __forceinline__ void init(int64_t ld_bytes, int64_t rows_valid, uint32_t wave, uint32_t lane)
    {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t q = wave * NL + i;
            const uint32_t row = 8 * q + lane / 8;
            const uint32_t chunk = (lane % 8) ^ ((row ^ (row >> 3)) & 7u);
            cb[i] = chunk * 16;
            base[i] = (int64_t)row < rows_valid ? (uint32_t)(row * ld_bytes + cb[i]) : OOB;
        }
    }
    // K-tile kt: bytes kt*128 .. +127 of each row (k_bytes = K * element size).
    // MASK: rows are only 4-byte aligned and K * element size need not be a
    // multiple of 16, so the vector that straddles the end of a row also holds
    // bytes of the next row; they are cleared here (the range check of the
    // buffer descriptor already zeroes whatever lies past the slice).
    __device__ __forceinline__ u32x4 load(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t k_bytes, uint32_t) const
    {
        const uint32_t kb0 = (uint32_t)kt * 128u;
        u32x4 x = load16(r, (base[i] != OOB && kb0 + cb[i] < k_bytes) ? base[i] + kb0 : OOB);
        if constexpr (MASK) {
            const int32_t rem = (int32_t)k_bytes - (int32_t)(kb0 + cb[i]); // bytes of the vector inside the row
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int32_t vb = rem - 4 * d;
                x[d] &= vb >= 4 ? 0xffffffffu : (vb <= 0 ? 0u : ((1u << (8 * vb)) - 1u));
            }
        }
        return x;
    }
    static __device__ __forceinline__ u32x4 frag(const char *tile, uint32_t row0, uint32_t ks, uint32_t lane)
    {
        return frag_read(tile, row0, ks, lane);
    }
};

// ---------------------------------------------------------------------------
// M/N-contiguous 16-bit operand: 64 K-rows x R values (2R bytes per row).
// Transfer i of wavefront w moves rows q*RPI .. +RPI-1 (q = w*NL + i, RPI =
// 512/R rows of 2R bytes); lane l fetches row q*RPI + l/CPR, logical chunk
// (l%CPR) ^ swz_t(row) (CPR = R/8 chunks per row), into physical chunk l%CPR.
// ---------------------------------------------------------------------------
template <int R, int NW> struct McStage {
    static_assert(R == 128 || R == 256, "transposed tile of 128 or 256 values");
    static constexpr int CPR = R / 8;
    static constexpr int RPI = 64 / CPR;
    static constexpr int NL = R / (8 * NW);
    static_assert(NL * 8 * NW == R, "whole 1 KiB transfers per wavefront");
    uint32_t base[NL]; // (k*ld + n) bytes at K-tile 0, or OOB
    uint32_t krow[NL]; // K-row within the K-tile

    __device__ __forceinline__ void init(int64_t ld_bytes, int64_t mn_valid, uint32_t wave, uint32_t lane)
    {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t q = wave * NL + i;
            const uint32_t k = q * RPI + lane / CPR;
            const uint32_t chunk = (lane % CPR) ^ swz_t(k);
            krow[i] = k;
            base[i] = (int64_t)(8 * chunk) < mn_valid ? (uint32_t)(k * ld_bytes + chunk * 16) : OOB;
        }
    }
    // K-tile kt: K-rows kt*64 .. +63 (k_rows = K; tile_step = 64 * ld bytes)
    __device__ __forceinline__ u32x4 load(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t k_rows,
                                          uint32_t tile_step) const
    {
        const uint32_t k0 = (uint32_t)kt * 64u;
        return load16(r, (base[i] != OOB && k0 + krow[i] < k_rows) ? base[i] + (uint32_t)kt * tile_step : OOB);
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

// Fragment that the MFMA sequence q = 0 .. MT*NT-1 (A fragment q / NT, B
// fragment q % NT) needs idx-th: A 0 with B 0, then B 1 .. NT-1 (with A 0),
// then A 1 .. MT-1.  A fragments are numbered 0..MT-1, B fragments MT.. .
// (A closed form, so that it folds to a constant in every unrolled loop.)
template <int MT, int NT> __device__ constexpr int first_use(int idx)
{
    return idx == 0 ? 0 : (idx <= NT ? MT + idx - 1 : idx - NT);
}

template <int MODE, int R, int NW> struct StageOf;
template <int R, int NW> struct StageOf<KC16, R, NW> { typedef KcStage<R, NW, false> type; };
template <int R, int NW> struct StageOf<KCD, R, NW> { typedef KcStage<R, NW, true> type; };
template <int R, int NW> struct StageOf<MC16, R, NW> { typedef McStage<R, NW> type; };

template <int T, int O, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
    __attribute__((amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4))) gemm_tiled(GemmParams p)
{
    constexpr int E = T == I8 ? 1 : 2;
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN; // wavefront tile
    constexpr int MT = WTM / 32, NT = WTN / 32;   // MFMA tiles per wavefront
    constexpr int ABYTES = BM * 128, STAGE = (BM + BN) * 128;
    static_assert(AMODE != MC16 || E == 2, "transposed operands are 16-bit");
    static_assert(BMODE != MC16 || E == 2, "transposed operands are 16-bit");
    typedef typename Mfma<T>::acc_t acc_t;
    typedef typename StageOf<AMODE, BM, NW>::type ATile;
    typedef typename StageOf<BMODE, BN, NW>::type BTile;
    constexpr int NA = ATile::NL, NB = BTile::NL;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave / WGN, wn = wave % WGN;
    const TileCoord tc = tile_of(p, blockIdx.x);
    const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;

    // Buffer descriptors cover this tile's part of each operand, from its first
    // row (K-contiguous) or column (M/N-contiguous) to the end of the batch slice.
    const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
    const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;
    const int64_t a_start = AMODE != MC16 ? m0 * p.lda * E : m0 * E;
    const int64_t b_start = BMODE != MC16 ? n0 * p.ldb * E : n0 * E;
    // The range check works per dword, and a slice may end inside one (4-byte
    // aligned rows, odd byte counts): the byte counts are rounded up to whole
    // dwords so that the straddling dword keeps its valid head; its tail is
    // cleared by the K-tail mask, and a dword never crosses a page.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_start, (uint32_t)((p.a_bytes - a_start + 3) & ~3ll));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_start, (uint32_t)((p.b_bytes - b_start + 3) & ~3ll));

    ATile ta;
    BTile tb;
    ta.init(p.lda * E, p.M - m0, wave, lane);
    tb.init(p.ldb * E, p.N - n0, wave, lane);
    // per-operand K extent and K-tile step for the loads
    const uint32_t a_kdim = AMODE != MC16 ? (uint32_t)p.K * E : (uint32_t)p.K;
    const uint32_t b_kdim = BMODE != MC16 ? (uint32_t)p.K * E : (uint32_t)p.K;
    const uint32_t a_step = (uint32_t)(64 * p.lda * E), b_step = (uint32_t)(64 * p.ldb * E);

    u32x4 sa[NA], sb[NB]; // the next K-tile between its global loads and its LDS writes
    auto load_one = [&](int c, int kt) {
        if (c < NA)
            sa[c] = ta.load(c, ra, kt, a_kdim, a_step);
        else
            sb[c - NA] = tb.load(c - NA, rb, kt, b_kdim, b_step);
    };
    auto store_one = [&](int c, char *stage) {
        if (c < NA)
            *reinterpret_cast<u32x4 *>(stage + (wave * NA + c) * 1024 + lane * 16) = sa[c];
        else
            *reinterpret_cast<u32x4 *>(stage + ABYTES + (wave * NB + (c - NA)) * 1024 + lane * 16) = sb[c - NA];
    };
    // The f-th fragment read of K-step ks, in the order of first use by the
    // MFMA sequence (fragment g: 0..MT-1 A rows, MT..MT+NT-1 B columns).
    auto read_one = [&](int f, const char *stage, int ks, u32x4 *af, u32x4 *bf) {
        f = first_use<MT, NT>(f);
        if (f < MT)
            af[f] = ATile::frag(stage, wm * WTM + f * 32, ks, lane);
        else
            bf[f - MT] = BTile::frag(stage + ABYTES, wn * WTN + (f - MT) * 32, ks, lane);
    };

    acc_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = acc_t{};

    const int nk = (int)(((int64_t)p.K * E + 127) / 128);
    constexpr int NLD = NA + NB, MN = MT * NT, NF = MT + NT;

    // Fragment registers: a double buffer over the K-steps, carried across
    // K-tiles (K-step 0 of the next K-tile is read while the last MFMAs of the
    // current one run).
    u32x4 af[2][MT], bfr[2][NT];

    if (nk > 0) {
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            load_one(c, 0);
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            store_one(c, smem);
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            load_one(c, 1);
        stage_barrier();
#pragma unroll
        for (int f = 0; f < NF; ++f)
            read_one(f, smem, 0, af[0], bfr[0]);
    }

    // Staging registers run one K-tile ahead of the LDS stages: in K-tile kt,
    // register c is written to the free stage (K-tile kt+1) and at once
    // reloaded with K-tile kt+2, so every global load has a whole K-tile of
    // MFMAs to arrive.  Near the end the same schedule runs on K-tiles that lie
    // wholly past K: the buffer range check turns their loads into zeros, so
    // the body needs no branches (branches around the loads make the compiler
    // drain the memory counters at every join).
    constexpr int SLOTS = 3 * MN; // MFMAs of K-steps 0-2 carry the copies
    for (int kt = 0; kt < nk; ++kt) {
        const char *cur = smem + (kt & 1) * STAGE;
        char *nxt = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
            const int c = ks & 1, n = c ^ 1;
#pragma unroll
            for (int q = 0; q < MN; ++q) {
                acc[q / NT][q % NT] = Mfma<T>::step(bfr[c][q % NT], af[c][q / NT], acc[q / NT][q % NT]);
                // fragments [q*NF/MN, (q+1)*NF/MN) of the next K-step
#pragma unroll
                for (int f = q * NF / MN; f < (q + 1) * NF / MN; ++f)
                    read_one(f, cur, ks + 1, af[n], bfr[n]);
                // staging registers [slot*NLD/SLOTS, (slot+1)*NLD/SLOTS): K-tile kt+1 to
                // LDS, then the loads of K-tile kt+2
                const int slot = ks * MN + q;
#pragma unroll
                for (int ci = slot * NLD / SLOTS; ci < (slot + 1) * NLD / SLOTS; ++ci) {
                    store_one(ci, nxt);
                    load_one(ci, kt + 2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // K-step 3: half of its MFMAs, the stage hand-over, then the other half
        // with the first fragment reads of K-tile kt+1.
#pragma unroll
        for (int q = 0; q < MN / 2; ++q) {
            acc[q / NT][q % NT] = Mfma<T>::step(bfr[1][q % NT], af[1][q / NT], acc[q / NT][q % NT]);
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_barrier();
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

    // Every wavefront is past the last barrier and reads no stage any more:
    // each parks its results in its own part of the stages.
    const char *Cb = p.C ? p.C + (int64_t)tc.b * p.stride_c * dt_bytes(O) : nullptr;
    char *Db = p.D + (int64_t)tc.b * p.stride_d * dt_bytes(O);
    constexpr int PARK = 32 * (32 * NT * 4 + 16);
    static_assert(NW * PARK <= 2 * STAGE, "parking area fits in the stages");
    store_staged<O, MT, NT>(p, acc, smem + wave * PARK, m0 + wm * WTM, n0 + wn * WTN, lane, Cb, Db);
}

} // namespace dmu
