// The tiled kernel (gemm_tiled).
//
// A workgroup of 8 wavefronts (WGM x WGN) computes a BM x BN tile of D; each
// wavefront owns an (BM/WGM) x (BN/WGN) block of 16 x 16 MFMA tiles.  K is
// walked in K-tiles of 128 bytes per row (64 fp16/bf16 or 128 int8 values),
// each two K-steps of the 16 x 16 instructions; 128 e4m3 values make one
// 16 x 16 x 128 step ("Tensor Cores, CUTLASS and CuTe" section 6.5: FP8's
// BK = 128 moves the bytes of BF16's BK = 64).  Three-level tiling
// (workgroup, wavefront, instruction) as in the
// "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough (sections 2-6) and
// "Tensor Cores, CUTLASS and CuTe" section 4.2, re-sized for 64-lane
// wavefronts, 160 KiB of LDS and two wavefronts per SIMD, so that one covers
// the other's memory waits.
//
// Data path of one K-tile:
//   global -> VGPR   buffer_load_dwordx4 through one buffer descriptor per
//                    operand: every out-of-range vector (rows past M/N, the K
//                    tail, K-tiles past K) reads as zeros without a branch.
//   VGPR -> LDS      ds_write_b128 into the other half of a double-buffered
//                    stage ring (the stage ring of "Tensor Cores, CUTLASS and
//                    CuTe" section 4.3, two stages deep here); one barrier per
//                    K-tile hands a stage over.
//   LDS -> VGPR      MFMA operand fragments: ds_read_b128 from a K-contiguous
//                    tile, or two ds_read_b64_tr_b16 from an M/N-contiguous
//                    16-bit tile (row-major B, column-major A) -- within each
//                    group of 16 lanes that instruction transposes the 16
//                    addressed 4-value rows (pinned by the layout probe).  This
//                    replaces the transposing shared-memory load of the pages
//                    (ldmatrix .trans, layout experiment section 5;
//                    walkthrough 5.3).
//
// A K-step's MFMAs cover the wavefront's MT x NT block of 16 x 16 tiles in two
// halves of its tile rows, each half walked column by column, issued as
// MFMA(srcA = B-fragment, srcB = A-fragment), i.e. D^T per tile (dmu_device.hpp).
//
// Register plan (the budget is 256 per lane with two wavefronts per SIMD):
// every fragment is single-buffered and is reloaded for the next K-step right
// after its last use in this one.  In the two-half order an A fragment's last
// use comes half a K-step before its next first use and a B fragment's last
// use comes a little less than half a K-step before, so every reload has a
// dozen or more MFMAs to arrive.  The K-tile body is an explicit issue
// schedule (scheduling barriers keep the order): after each MFMA come the
// fragment reads it frees registers for, and a share of the staging copies
// (the next K-tile's LDS writes, each followed by the global load of the
// K-tile after it into the same registers).
#pragma once

#include "dmu_device.hpp"

#include <type_traits>

// LDS-poisoning debug build (compiled with DMU_LDS_POISON=1; never the product
// library): right after the barrier that retires a stage, each wavefront
// overwrites its own staging slots of that stage with all-ones bytes (NaN in
// fp16, bf16 and e4m3, -1 in int8), long before the next K-tile's data lands
// there.  A fragment read that strayed past its barrier would then feed the
// poison into D, so parity of this build with the product build bit for bit
// shows that every stage is read only inside its window.
#ifndef DMU_LDS_POISON
#define DMU_LDS_POISON 0
#endif

namespace dmu {

// ---------------------------------------------------------------------------
// Global -> register loads.  Each operand has one buffer descriptor, from this
// tile's first row (K-contiguous) or column (M/N-contiguous) to the end of the
// batch slice; a load's address is that base + a per-lane offset (one register
// per operand) + a uniform offset in the instruction's scalar offset field
// (transfer and K-tile).  The range check covers both offsets, so rows or
// K-rows past the matrix read as zeros, and so does a lane offset of OOB.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// K-contiguous operand (A row-major, B column-major): R rows of one K-tile
// (128 bytes), the eight 16-byte chunks of row r permuted by XOR with r mod 8
// (measured on gfx950: conflict-free for the 16 x 16 fragment reads, while a
// padded pitch is not).  Row r0 + (l % 16) of a fragment has r mod 8 = l mod 8
// for every 16-aligned r0, so each fragment address is one of two per-lane
// bases (K-step 0 or 1) plus a constant.
// ---------------------------------------------------------------------------
template <int R, int NW, bool MASK> struct KcTile {
    static constexpr int NL = R / (8 * NW); // 1 KiB transfers per wavefront
    static_assert(NL * 8 * NW == R, "whole 1 KiB transfers per wavefront");
    static constexpr uint32_t BYTES = R * 128;
    uint32_t voff;  // lane offset within a transfer: row l / 8, chunk l % 8
    uint32_t cb;    // byte of that chunk within a K-tile row
    uint32_t wlane; // LDS offset of this lane's 16 bytes within a transfer
    uint32_t first; // byte offset of the wavefront's first row
    uint32_t xstep; // bytes between the first rows of consecutive transfers
    uint32_t tm[MASK ? 4 : 1]; // MASK: this lane's byte mask of its chunk in the K-tile holding the row end

    // MASK: rows are only 4-byte aligned and K * element size need not be a
    // multiple of 16, so in the K-tile that holds the end of the rows, the vector
    // that straddles a row's end also holds bytes of the next row.  Which bytes
    // are this lane's own depends only on its chunk, the same in every row.
    __device__ __forceinline__ void init_mask(uint32_t k_bytes)
    {
        if constexpr (MASK) {
            const uint32_t kl = (k_bytes - 1u) / 128u; // the K-tile holding the row end
            const int32_t rem = (int32_t)k_bytes - (int32_t)(kl * 128u + cb);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int32_t vb = rem - 4 * d;
                tm[d] = vb >= 4 ? 0xffffffffu : (vb <= 0 ? 0u : ((1u << (8 * vb)) - 1u));
            }
        }
    }

    // Transfer i of wavefront w moves rows 8q .. 8q+7 (q = w NL + i) into LDS
    // bytes 1024 q .. +1023: lane l carries row 8q + l / 8, chunk l % 8 (eight
    // consecutive lanes read one 128-byte row segment in order), to physical
    // chunk (l % 8) ^ (l / 8).
    __device__ __forceinline__ void init(int64_t ld_bytes, uint32_t wave, uint32_t lane)
    {
        cb = (lane & 7u) * 16;
        voff = (lane >> 3) * (uint32_t)ld_bytes + cb;
        wlane = (lane >> 3) * 128 + (((lane & 7u) ^ (lane >> 3)) << 4);
        first = 8 * wave * NL * (uint32_t)ld_bytes;
        xstep = 8 * (uint32_t)ld_bytes;
    }
    // K-tile kt: bytes kt*128 .. +127 of each row (k_bytes = K * element size).
    __device__ __forceinline__ u32x4 load(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t k_bytes) const
    {
        const uint32_t kb0 = (uint32_t)kt * 128u;
        return load16s(r, kb0 + cb < k_bytes ? voff : OOB, first + (uint32_t)i * xstep + kb0);
    }
    // The data of K-tile kt to LDS.  MASK: in the K-tile holding the row end,
    // the bytes past it (the next row's) are cleared here, where the load has
    // long completed (clearing them right after the load would make the
    // wavefront wait for it there); the other K-tiles keep every byte.  (Before,
    // the mask was derived in every K-tile from the bytes left: 5000 x 3000 x
    // 2050 fp16, rows of 4100 bytes, 65.7 -> 64.3 us with the mask taken once,
    // same bits.)
    __device__ __forceinline__ void store(int i, char *tile, uint32_t wave, uint32_t, u32x4 v, int kt,
                                          uint32_t k_bytes) const
    {
        if constexpr (MASK) {
            const uint32_t keep = (uint32_t)kt * 128u + 128u <= k_bytes ? ~0u : 0u;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                v[d] &= tm[d] | keep;
        }
        *reinterpret_cast<u32x4 *>(tile + (wave * NL + i) * 1024 + wlane) = v;
    }
    // Transfer i's 16 bytes of this lane, unmasked (the poisoning debug build).
    __device__ __forceinline__ void store_raw(int i, char *tile, uint32_t wave, u32x4 v) const
    {
        *reinterpret_cast<u32x4 *>(tile + (wave * NL + i) * 1024 + wlane) = v;
    }
    // Rows [r0, r0 + 16) (r0 a multiple of 16), K-step ks (0, 1): lane l reads
    // row r0 + l % 16, logical bytes 64 ks + 16 (l / 16) .. +15 of the K-tile.
    static __device__ __forceinline__ u32x4 frag(const char *tile, uint32_t r0, uint32_t ks, uint32_t lane)
    {
        const uint32_t chunk = (4 * ks + (lane >> 4)) ^ (lane & 7u);
        return *reinterpret_cast<const u32x4 *>(tile + (r0 + (lane & 15u)) * 128 + chunk * 16);
    }
};

// ---------------------------------------------------------------------------
// M/N-contiguous 16-bit operand (B row-major, A column-major): the 64 K-rows of
// a K-tile, R values (2R bytes) each, row pitch 2R + 32 bytes, K-rows with bit
// 3 clear in a first region and those with bit 3 set in a second one that
// starts 128 bytes past a multiple of 256.  A transposing read by 16 lanes
// covers four consecutive K-rows x 32 bytes, which the 32-byte row shift puts
// on four different 32-byte bank groups; the two 16-lane groups that read
// K-rows k and k + 8 land in opposite 128-byte halves (measured on gfx950:
// conflict-free; without the region split, two-way conflicts).  Each fragment
// address is one per-lane base plus a constant.
// ---------------------------------------------------------------------------
template <int R> __device__ __forceinline__ constexpr uint32_t mc_row_off(uint32_t k)
{
    constexpr uint32_t P = 2 * R + 32;
    return ((k >> 3) & 1u) * (32 * P + 128) + ((k & 7u) | ((k >> 4) << 3)) * P;
}

template <int R, int NW> struct McTile {
    static_assert(R == 128 || R == 256, "transposed tile of 128 or 256 values");
    static constexpr int CPR = R / 8;   // 16-byte chunks per K-row
    static constexpr int RPI = 64 / CPR; // K-rows per 1 KiB transfer
    static constexpr int NL = R / (8 * NW);
    static_assert(NL * 8 * NW == R, "whole 1 KiB transfers per wavefront");
    static constexpr uint32_t BYTES = 64 * (2 * R + 32) + 128;
    uint32_t voff;     // K-row l / CPR, chunk l % CPR; OOB for columns past N
    uint32_t wofs[NL]; // LDS byte offset of each staging write
    uint32_t first;    // byte offset of the wavefront's first K-row
    uint32_t xstep;    // bytes between the first K-rows of consecutive transfers
    uint32_t kstep;    // bytes per K-tile (64 K-rows)

    // Transfer i of wavefront w moves K-rows q RPI .. +RPI-1 (q = w NL + i):
    // lane l carries K-row q RPI + l / CPR, chunk l % CPR.
    __device__ __forceinline__ void init(int64_t ld_bytes, int64_t mn_valid, uint32_t wave, uint32_t lane)
    {
        const uint32_t chunk = lane % CPR;
        voff = (int64_t)(8 * chunk) < mn_valid ? (lane / CPR) * (uint32_t)ld_bytes + chunk * 16 : OOB;
        first = wave * NL * RPI * (uint32_t)ld_bytes;
        xstep = RPI * (uint32_t)ld_bytes;
        kstep = 64 * (uint32_t)ld_bytes;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            wofs[i] = mc_row_off<R>((wave * NL + i) * RPI + lane / CPR) + chunk * 16;
    }
    // K-tile kt: K-rows kt*64 .. +63; K-rows past K lie past the slice end.
    __device__ __forceinline__ u32x4 load(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t) const
    {
        return load16s(r, voff, first + (uint32_t)i * xstep + (uint32_t)kt * kstep);
    }
    __device__ __forceinline__ void store(int i, char *tile, uint32_t, uint32_t, u32x4 v, int, uint32_t) const
    {
        *reinterpret_cast<u32x4 *>(tile + wofs[i]) = v;
    }
    __device__ __forceinline__ void store_raw(int i, char *tile, uint32_t, u32x4 v) const
    {
        *reinterpret_cast<u32x4 *>(tile + wofs[i]) = v;
    }
    // Columns [c0, c0 + 16), K-step ks: lane l gets column c0 + l % 16 and
    // k = 32 ks + 8 (l / 16) + 0..7, by two transposing reads (k .. k+3, then
    // k+4 .. k+7).  Lane j of each 16-lane group g addresses
    // X[32 ks + 8 g + j / 4][c0 + 4 (j % 4)]; the probe pins that lane i of the
    // group then receives X[32 ks + 8 g .. +3][c0 + i].
    static __device__ __forceinline__ u32x4 frag(const char *tile, uint32_t c0, uint32_t ks, uint32_t lane)
    {
        constexpr uint32_t P = 2 * R + 32;
        const uint32_t g = lane >> 4, j = lane & 15u;
        const uint32_t k = 32 * ks + 8 * g + (j >> 2);
        const uint32_t a0 = mc_row_off<R>(k) + (c0 + 4 * (j & 3u)) * 2;
        const uint32_t a1 = a0 + 4 * P; // k + 4: same region, four rows on
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(tile + a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(tile + a1));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
    // Columns [c0, c0 + 16), keys of K-step kk (32 keys) in the order that the
    // 16 x 16 accumulator of a preceding product leaves them in (lane l owns
    // rows 4 (l / 16) + 0..3 of each 16-row tile): lane l gets column c0 + l % 16
    // at k = 32 kk + 4 (l / 16) + 0..3 and 32 kk + 16 + 4 (l / 16) + 0..3.  So the
    // accumulators of two adjacent 16-key tiles, packed, are the other operand
    // of the same instruction, with no data movement.
    static __device__ __forceinline__ u32x4 frag_split(const char *tile, uint32_t c0, uint32_t kk, uint32_t lane)
    {
        constexpr uint32_t P = 2 * R + 32;
        const uint32_t g = lane >> 4, j = lane & 15u;
        const uint32_t k = 32 * kk + 4 * g + (j >> 2);
        const uint32_t a0 = mc_row_off<R>(k) + (c0 + 4 * (j & 3u)) * 2;
        const uint32_t a1 = a0 + 8 * P; // k + 16: same region, eight region rows on
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(tile + a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(tile + a1));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
};

// ---------------------------------------------------------------------------
// M/N-contiguous 8-bit operand (column-major A or row-major B, int8 or e4m3):
// the 128 K-rows of a
// K-tile, R bytes each, K-row k at byte k (R + 16) + 128 (k / 16).  A fragment
// (16 columns, 16 consecutive k of one 64-k half) is two ds_read_b64_tr_b8:
// within each group of 16 lanes, if lane j addresses X[k0 + j / 2][c0 + 8 (j %
// 2) .. +7], lane i receives X[k0 .. k0 + 7][c0 + i] (pinned by the layout
// probe).
//   reads   lane l (group g = l / 16) reads K-row 64 h + 16 g + (l % 16) / 2 (+ 8
//           for the second read): the 16-byte pitch excess puts the eight K-rows
//           of a group in eight different 16-byte slots of a 256-byte bank line,
//           and the 128 bytes added after every 16 K-rows move the next group
//           (16 K-rows on) to the other eight slots, so lanes l and l + 16
//           never share a bank; only lanes 32 apart do.
//   writes  eight consecutive lanes put 128 consecutive bytes of one K-row.
// Every offset is a per-lane base plus a constant, as in the unswizzled tile.
// ---------------------------------------------------------------------------
typedef int i32x2 __attribute__((ext_vector_type(2)));
template <int R, int NW> struct McTile8 {
    static_assert(R == 128 || R == 256, "transposed tile of 128 or 256 values");
    static constexpr int P = R + 16;      // K-row pitch within a block of 16 K-rows
    static constexpr int CPR = R / 16;    // 16-byte chunks per K-row
    static constexpr int RPI = 64 / CPR;  // K-rows per 1 KiB transfer
    static constexpr int NL = R / (8 * NW);
    static_assert(NL * 8 * NW == R, "whole 1 KiB transfers per wavefront");
    static constexpr uint32_t BYTES = 128 * P + 8 * 128;
    static __device__ __forceinline__ uint32_t row(uint32_t k) { return k * P + (k >> 4) * 128; }
    uint32_t voff;     // K-row l / CPR, chunk l % CPR; OOB for columns past N
    uint32_t wofs[NL]; // LDS byte offset of each staging write
    uint32_t first;    // byte offset of the wavefront's first K-row
    uint32_t xstep;    // bytes between the first K-rows of consecutive transfers
    uint32_t kstep;    // bytes per K-tile (128 K-rows)
    __device__ __forceinline__ void init(int64_t ld_bytes, int64_t mn_valid, uint32_t wave, uint32_t lane)
    {
        const uint32_t chunk = lane % CPR;
        voff = (int64_t)(16 * chunk) < mn_valid ? (lane / CPR) * (uint32_t)ld_bytes + chunk * 16 : OOB;
        first = wave * NL * RPI * (uint32_t)ld_bytes;
        xstep = RPI * (uint32_t)ld_bytes;
        kstep = 128 * (uint32_t)ld_bytes;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            wofs[i] = row((wave * NL + i) * RPI + lane / CPR) + chunk * 16;
    }
    __device__ __forceinline__ u32x4 load(int i, __amdgpu_buffer_rsrc_t r, int kt, uint32_t) const
    {
        return load16s(r, voff, first + (uint32_t)i * xstep + (uint32_t)kt * kstep);
    }
    __device__ __forceinline__ void store(int i, char *tile, uint32_t, uint32_t, u32x4 v, int, uint32_t) const
    {
        *reinterpret_cast<u32x4 *>(tile + wofs[i]) = v;
    }
    __device__ __forceinline__ void store_raw(int i, char *tile, uint32_t, u32x4 v) const
    {
        *reinterpret_cast<u32x4 *>(tile + wofs[i]) = v;
    }
    // Columns [c0, c0 + 16), k = 64 h + 16 (l / 16) + 0..15 (h: the 64-k half of
    // the K-tile -- the K-step of the int8 instruction, or one of the two
    // 16-byte operand halves of the e4m3 one): lane l gets column c0 + l % 16.
    // The second read's K-rows (k + 8) lie in the same block of 16.
    static __device__ __forceinline__ u32x4 frag(const char *tile, uint32_t c0, uint32_t h, uint32_t lane)
    {
        const uint32_t g = lane >> 4, j = lane & 15u;
        const uint32_t a0 = row(64 * h + 16 * g + (j >> 1)) + c0 + 8 * (j & 1u);
        const uint32_t a1 = a0 + 8 * P;
        const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(tile + a0));
        const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(tile + a1));
        return u32x4{(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
    }
};

template <int MODE, int R, int NW> struct TileOf;
template <int R, int NW> struct TileOf<KC16, R, NW> { typedef KcTile<R, NW, false> type; };
template <int R, int NW> struct TileOf<KCD, R, NW> { typedef KcTile<R, NW, true> type; };
template <int R, int NW> struct TileOf<MC16, R, NW> { typedef McTile<R, NW> type; };
template <int R, int NW> struct TileOf<MC8, R, NW> { typedef McTile8<R, NW> type; };

// ---------------------------------------------------------------------------
// Epilogue through LDS for 16 x 16 tiles: each 16-row stripe of the
// wavefront's results is parked in its own LDS area and read back
// row-contiguous, so that every store instruction writes whole rows of 16 NT
// values, with the fused epilogue (scales, bias, C, activation), RNE
// conversion and M/N masking on the way out.
// ---------------------------------------------------------------------------
// Geometry of the parked stripes.  A stripe is 16 rows of 16 NT accumulator
// columns (fp32 / int32) per wavefront, rows of ROWB bytes without padding,
// the 16-byte chunks of row r permuted by XOR with r (mod the chunks per row).
//
// LDS bank rules: the conflict counters of the K loop's staging writes and
// fragment reads and of several park layouts are fitted by a ds_write_b128
// served 8 consecutive lanes per cycle over 32 banks of 4 bytes, and a
// ds_read_b128 served 16 lanes per cycle over 64 banks in quad-structured
// groups -- lanes {0-3, 12-15, 20-23, 24-27}, and the groups obtained from it
// by flipping lane bits 2 and 5.
//   writes  lane l puts row l % 16, chunk 4 ni + l / 16: the 8 lanes of a
//           write group hold rows r .. r+7 at one chunk, which the XOR
//           spreads over the 8 chunk slots of 128 bytes;
//   reads   lane l takes row l / CH + RPI it, chunk l % CH: a read group
//           spans two adjacent rows 2j, 2j + 1 (the same XOR above bit 0),
//           and takes chunks with bit 2 = bit 3 from one and bit 2 != bit 3
//           from the other, which the XOR keeps apart.
// Each aligned block of CH lanes reads (and stores to D) one whole row, so
// every store instruction writes whole rows with consecutive lanes.
template <int NT> struct Park {
    static_assert(NT == 2 || NT == 4 || NT == 8, "wavefront tiles of 32, 64 or 128 columns");
    static constexpr int COLS = 16 * NT;
    static constexpr int ROWB = COLS * 4;     // bytes per parked row
    static constexpr int CH = COLS / 4;       // 16-byte chunks per row: 8, 16 or 32
    static constexpr int RPI = 64 / CH;       // rows per read instruction
    static constexpr int ITS = 16 / RPI;      // reads per stripe
    static constexpr int RSTEP = RPI;         // a lane's row step between reads
    static constexpr int BYTES = 16 * ROWB;
    static __device__ __forceinline__ uint32_t addr(uint32_t r, uint32_t chunk)
    {
        return r * ROWB + ((chunk ^ (r & (CH - 1))) << 4);
    }
    static __device__ __forceinline__ uint32_t rd_row(uint32_t l) { return l / CH; }
    static __device__ __forceinline__ uint32_t rd_chunk(uint32_t l) { return l % CH; }
    // Stripe mi: lane l's accumulator tile ni holds row l % 16, columns 16 ni + 4 (l / 16) ..
    template <class AccT, int MT>
    static __device__ __forceinline__ void put(char *lds, const AccT (&acc)[MT][NT], int mi, uint32_t lane)
    {
        typedef typename std::remove_const<typename std::remove_reference<decltype(acc[0][0][0])>::type>::type st;
        typedef st st4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
            st4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = acc[mi][ni][e];
            *reinterpret_cast<st4 *>(lds + addr(lane & 15u, 4 * ni + (lane >> 4))) = v;
        }
    }
    // Read it of a stripe: this lane's 4 values of row rd_row(l) + RSTEP it.
    template <class st4>
    static __device__ __forceinline__ st4 get(const char *lds, int it, uint32_t lane)
    {
        return *reinterpret_cast<const st4 *>(lds + addr(rd_row(lane) + RSTEP * it, rd_chunk(lane)));
    }
};

// One vector of D: a streaming (non-temporal) store -- D is not read again by
// this kernel, and all tiles write it in one burst at the end (4096^3 bf16:
// 113 -> 110 us; batched 4096 x 4096 x 128 fp32: 485 -> 386 us) -- or, when D's
// rows start inside a 128-byte line, a store written through this XCD's L2
// (cache policy SC1, i.e. a relaxed store at device scope, 8 bytes at a time):
// two tiles then write the parts of a shared line, which as streaming stores
// leave for memory as separate partial lines (5000 x 3000 x 2050 fp16: 68.8 us
// against 66.4 us with plain stores), while plain stores leave every line of D
// dirty in the L2s for the write-back at the end of the kernel (66.2 -> 65.2 us
// written through, interleaved in one process; same bits).
template <bool NTS, class V> __device__ __forceinline__ void store_d(V *dst, const V &v)
{
    if constexpr (NTS) {
        __builtin_nontemporal_store(v, dst);
    } else {
        static_assert(sizeof(V) % 8 == 0, "D vectors are 8 or 16 bytes");
        typedef uint64_t w_t __attribute__((ext_vector_type(sizeof(V) / 8)));
        const w_t w = __builtin_bit_cast(w_t, v);
        uint64_t *d = reinterpret_cast<uint64_t *>(dst);
#pragma unroll
        for (int i = 0; i < (int)(sizeof(V) / 8); ++i)
            __hip_atomic_store(d + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// A wavefront block wholly inside D (every row < M, every 4-column vector
// < N and aligned), with the epilogue's form fixed at compile time.
template <int O, int MT, int NT, bool HAS_C, bool EPI, int ACT, bool NTS, class AccT>
__device__ __forceinline__ void store_interior(const GemmParams &p, const AccT (&acc)[MT][NT], char *lds,
                                               int64_t m_base, uint32_t lane, int64_t n, const char *Cb,
                                               char *Db, const EpiPtrs &ep)
{
    typedef Park<NT> K;
    typedef typename Out<O>::t ot;
    typedef typename std::remove_const<typename std::remove_reference<decltype(acc[0][0][0])>::type>::type st;
    typedef st st4 __attribute__((ext_vector_type(4)));
    typedef ot ov4 __attribute__((ext_vector_type(4)));
    const uint32_t r0 = K::rd_row(lane);
    float csv[4] = {1.0f, 1.0f, 1.0f, 1.0f}, bv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, rsv[MT][K::ITS];
    if constexpr (EPI) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            csv[e] = ep.cs ? ep.cs[n + e] : 1.0f;
            bv[e] = ep.bias ? ep.bias[n + e] : 0.0f;
        }
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int it = 0; it < K::ITS; ++it)
                rsv[mi][it] = ep.rs ? ep.rs[m_base + mi * 16 + K::RSTEP * it + r0] : 1.0f;
    }
    const int64_t rel = (m_base + r0) * p.ldd + n; // this lane's first element of D
    ot *D0 = reinterpret_cast<ot *>(Db) + rel;
    const ot *C0 = HAS_C ? reinterpret_cast<const ot *>(Cb) + (m_base + r0) * p.ldc + n : nullptr;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
        ov4 c[K::ITS];
        if constexpr (HAS_C) {
#pragma unroll
            for (int it = 0; it < K::ITS; ++it)
                c[it] = *reinterpret_cast<const ov4 *>(C0 + (int64_t)(mi * 16 + K::RSTEP * it) * p.ldc);
        }
        K::put(lds, acc, mi, lane);
#pragma unroll
        for (int it = 0; it < K::ITS; ++it) {
            const st4 v = K::template get<st4>(lds, it, lane);
            ov4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = epi_one<O>(EPI, ACT, v[e], EPI ? rsv[mi][it] : 1.0f, csv[e], bv[e], HAS_C,
                                  HAS_C ? c[it][e] : ot{});
            store_d<NTS>(reinterpret_cast<ov4 *>(D0 + (int64_t)(mi * 16 + K::RSTEP * it) * p.ldd), o);
        }
    }
}

// A plain block (no C, no epilogue operations) that crosses the M or N edge:
// rows past M are skipped and a vector that crosses N is stored element by
// element, with no other per-row decisions.
template <int O, int MT, int NT, class AccT>
__device__ __forceinline__ void store_edge_plain(const GemmParams &p, const AccT (&acc)[MT][NT], char *lds,
                                                 int64_t m_base, uint32_t lane, int64_t n, char *Db)
{
    typedef Park<NT> K;
    typedef typename Out<O>::t ot;
    typedef typename std::remove_const<typename std::remove_reference<decltype(acc[0][0][0])>::type>::type st;
    typedef st st4 __attribute__((ext_vector_type(4)));
    typedef ot ov4 __attribute__((ext_vector_type(4)));
    const uint32_t r0 = K::rd_row(lane);
    const bool vec = p.d_vec4 && n + 3 < p.N;
    const int nv = n >= p.N ? 0 : (p.N - n < 4 ? (int)(p.N - n) : 4); // valid elements of this lane's vector
    ot *D0 = reinterpret_cast<ot *>(Db) + (m_base + r0) * p.ldd + n;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
        K::put(lds, acc, mi, lane);
#pragma unroll
        for (int it = 0; it < K::ITS; ++it) {
            const st4 v = K::template get<st4>(lds, it, lane);
            if (m_base + mi * 16 + K::RSTEP * it + r0 >= p.M)
                continue;
            ov4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = epi_one<O>(0, 0, v[e], 1.0f, 1.0f, 0.0f, false, ot{});
            ot *d = D0 + (int64_t)(mi * 16 + K::RSTEP * it) * p.ldd;
            if (vec) {
                if (p.d_nt)
                    store_d<true>(reinterpret_cast<ov4 *>(d), o);
                else
                    store_d<false>(reinterpret_cast<ov4 *>(d), o);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < nv)
                        d[e] = o[e];
            }
        }
    }
}

// A wavefront's MT x NT block of accumulator tiles to D, through the LDS
// park (lds: this wavefront's PARK bytes), with the fused epilogue.
template <int O, int MT, int NT, class AccT>
__device__ __forceinline__ void store_staged(const GemmParams &p, const AccT (&acc)[MT][NT], char *lds,
                                             int64_t m_base, int64_t n_base, uint32_t lane, const char *Cb,
                                             char *Db, const EpiPtrs &ep)
{
    typedef Park<NT> K;
    typedef typename Out<O>::t ot;
    typedef typename std::remove_const<typename std::remove_reference<decltype(acc[0][0][0])>::type>::type st;
    typedef st st4 __attribute__((ext_vector_type(4)));
    typedef ot ov4 __attribute__((ext_vector_type(4)));
    // On the way out lane l always handles the same four columns (n_base +
    // 4 rd_chunk(l) ..) and, in stripe mi and store it, row 16 mi + RSTEP it + rd_row(l).
    const uint32_t col = K::rd_chunk(lane) * 4, r0 = K::rd_row(lane);
    const int64_t n = n_base + col;

    // A block wholly inside D with 4-element vectors legal needs no per-row
    // decisions.  The epilogue's form (C or not, scales and bias or not,
    // activation) is uniform, so it is decided once here and each form is a
    // branch-free instantiation: per-element branches cost more than the
    // arithmetic (the plain 4096^3 bf16 product: 112 -> 104 us; the batched
    // 4096 x 4096 x 128 product, 32 tiles per compute unit: 524 -> 427 us).
    if (p.d_vec4 && m_base + 16 * MT <= p.M && n_base + K::COLS <= p.N) {
        const int form = (Cb ? 1 : 0) | (p.epi ? 2 : 0);
        // plain stores for the plain form when D's rows start inside a line
        if (form == 0 && p.act == 0 && !p.d_nt)
            return store_interior<O, MT, NT, false, false, 0, false>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        switch (form * 3 + (p.act == 1 ? 1 : p.act == 2 ? 2 : 0)) {
        case 0: return store_interior<O, MT, NT, false, false, 0, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 1: return store_interior<O, MT, NT, false, false, 1, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 2: return store_interior<O, MT, NT, false, false, 2, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 3: return store_interior<O, MT, NT, true, false, 0, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 4: return store_interior<O, MT, NT, true, false, 1, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 5: return store_interior<O, MT, NT, true, false, 2, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 6: return store_interior<O, MT, NT, false, true, 0, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 7: return store_interior<O, MT, NT, false, true, 1, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 8: return store_interior<O, MT, NT, false, true, 2, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 9: return store_interior<O, MT, NT, true, true, 0, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        case 10: return store_interior<O, MT, NT, true, true, 1, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        default: return store_interior<O, MT, NT, true, true, 2, true>(p, acc, lds, m_base, lane, n, Cb, Db, ep);
        }
    }
    if (!Cb && !p.epi && !p.act)
        return store_edge_plain<O, MT, NT>(p, acc, lds, m_base, lane, n, Db);

    // Any other block: per-row and per-element decisions, one row group per
    // iteration (a loop rather than unrolled, to keep this rarely taken path
    // small).  Row scales are fetched up front: fetched in the loop they would
    // stall every iteration.
    const bool vec = p.d_vec4 && n + 3 < p.N; // whole 4-element vector inside D (and aligned)
    float rsv[MT][K::ITS], csv[4], bv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool in = n + e < p.N;
        csv[e] = ep.cs && in ? ep.cs[n + e] : 1.0f;
        bv[e] = ep.bias && in ? ep.bias[n + e] : 0.0f;
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int it = 0; it < K::ITS; ++it) {
            const int64_t m = m_base + mi * 16 + K::RSTEP * it + r0;
            rsv[mi][it] = ep.rs && m < p.M ? ep.rs[m] : 1.0f;
        }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
        K::put(lds, acc, mi, lane);
#pragma nounroll
        for (int it = 0; it < K::ITS; ++it) {
            float rs = rsv[mi][0];
#pragma unroll
            for (int i = 1; i < K::ITS; ++i)
                rs = it == i ? rsv[mi][i] : rs;
            const uint32_t row = K::RSTEP * it + r0;
            const st4 v = K::template get<st4>(lds, it, lane);
            const int64_t m = m_base + mi * 16 + row;
            if (m >= p.M)
                continue;
            const ot *Crow = Cb ? reinterpret_cast<const ot *>(Cb) + m * p.ldc : nullptr;
            ot *Drow = reinterpret_cast<ot *>(Db) + m * p.ldd;
            ov4 c = {}, o;
            if (Crow) {
                if (vec)
                    c = *reinterpret_cast<const ov4 *>(Crow + n);
                else
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N)
                            c[e] = Crow[n + e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = epi_one<O>(p.epi, p.act, v[e], rs, csv[e], bv[e], Crow != nullptr, c[e]);
            if (vec) {
                if (p.d_nt)
                    store_d<true>(reinterpret_cast<ov4 *>(Drow + n), o);
                else
                    store_d<false>(reinterpret_cast<ov4 *>(Drow + n), o);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < p.N)
                        Drow[n + e] = o[e];
            }
        }
    }
}

// This batch slice's epilogue vectors.
__device__ __forceinline__ EpiPtrs epi_ptrs(const GemmParams &p, int64_t b)
{
    EpiPtrs e;
    e.rs = p.rs ? p.rs + b * p.stride_rs : nullptr;
    e.cs = p.cs ? p.cs + b * p.stride_cs : nullptr;
    e.bias = p.bias ? p.bias + b * p.stride_bias : nullptr;
    return e;
}

// One workgroup's tile of the product: the constants of a configuration, the
// main loop over a range of K-tiles, the epilogue and (for the stream-K
// kernel) the exchange of partial sums.
template <int T, int O, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE> struct Tiled {
    static constexpr bool F8 = T == E4M3;           // one 16 x 16 x 128 MFMA per K-tile and tile
    static constexpr int E = (T == I8 || F8) ? 1 : 2;
    static constexpr int FH = F8 ? 2 : 1;           // 16-byte fragment halves an MFMA reads
    static constexpr int NW = WGM * WGN;
    static_assert(NW == 8 || NW == 4, "eight wavefronts (two per SIMD) or four (one per SIMD)");
    // Four wavefronts: 128 x 128 wavefront tiles, whose 256 accumulator
    // registers live in the AGPRs (one wavefront per SIMD holds 512 registers);
    // the MFMAs update them in place, and the first K-step of a range writes
    // them from a zero accumulator operand (no initialisation of the
    // accumulators precedes the main loop).
    static constexpr bool AG = NW == 4;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN; // wavefront tile
    static constexpr int MT = WTM / 16, NT = WTN / 16;   // MFMA tiles per wavefront
    static constexpr int MN = MT * NT;
    static_assert(MT % 2 == 0, "a K-step runs in two halves of the tile rows");
    static_assert(AMODE != MC16 || E == 2, "transposed operands are 16-bit");
    static_assert(BMODE != MC16 || E == 2, "transposed operands are 16-bit");
    static_assert(BMODE != MC8 || E == 1, "the 8-bit transposed layout takes 8-bit operands");
    static_assert(AMODE != MC8 || E == 1, "the 8-bit transposed layout takes 8-bit operands");
    static_assert(!F8 || MN <= 16, "e4m3 fragments (8 registers per tile) fit beside the accumulators");
    static_assert(!AG || !F8, "the four-wavefront tile takes the 16-bit and int8 instructions");
    typedef typename Mfma<T>::acc_t acc_t;
    typedef typename TileOf<AMODE, BM, NW>::type ATile;
    typedef typename TileOf<BMODE, BN, NW>::type BTile;
    static constexpr int NA = ATile::NL, NB = BTile::NL;
    // Prefetch depth: K-tiles in flight in staging registers.  Two where the
    // registers allow (every configuration but 256 x 256, whose accumulators
    // and fragments leave room for one set): the loads of K-tile kt+3 go out
    // while K-tile kt+1 is written to LDS, which doubles the bytes in flight
    // per compute unit.
    static constexpr int PD = (BM * BN < 256 * 256) ? 2 : 1;
    static constexpr uint32_t ABYTES = (ATile::BYTES + 255) & ~255u,
                              STAGE = (ABYTES + BTile::BYTES + 255) & ~255u;
    static constexpr int PARK = Park<NT>::BYTES; // per wavefront, epilogue
    static_assert(NW * PARK <= 2 * STAGE, "parking area fits in the stages");
    static constexpr uint32_t PARTIAL_BYTES = NW * MN * 1024; // one tile's accumulators

    // Staging registers, owned by the caller so that the persistent kernel can
    // load the next tile's first K-tile before the current tile's epilogue.
    struct Staging {
        u32x4 sa[PD][NA];
        u32x4 sb[PD][NB];
    };
    // Load K-tile kb of tile tc into staging set 0 (what the main loop's
    // prologue would load first) -- or, with n > 1, K-tiles kb .. kb + n - 1
    // into sets 0 .. n - 1 (n <= PD: a whole short K range, for short_loop).
    static __device__ __forceinline__ void prefetch(const GemmParams &p, const TileCoord tc, int kb, Staging &st,
                                                    uint32_t tid, int n = 1)
    {
        const uint32_t lane = tid & 63u;
        const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
        const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
        const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;
        const int64_t a_start = (AMODE == MC16 || AMODE == MC8) ? m0 * E : m0 * p.lda * E;
        const int64_t b_start = (BMODE == MC16 || BMODE == MC8) ? n0 * E : n0 * p.ldb * E;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_start, (uint32_t)((p.a_bytes - a_start + 3) & ~3ll));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_start, (uint32_t)((p.b_bytes - b_start + 3) & ~3ll));
        ATile ta;
        BTile tb;
        if constexpr (AMODE == MC16 || AMODE == MC8)
            ta.init(p.lda * E, p.M - m0, wave, lane);
        else
            ta.init(p.lda * E, wave, lane);
        if constexpr (BMODE == MC16 || BMODE == MC8)
            tb.init(p.ldb * E, p.N - n0, wave, lane);
        else
            tb.init(p.ldb * E, wave, lane);
        const uint32_t k_bytes = (uint32_t)p.K * E;
#pragma unroll
        for (int set = 0; set < PD; ++set) {
            if (set > 0 && set >= n)
                break;
#pragma unroll
            for (int c = 0; c < NA; ++c)
                st.sa[set][c] = ta.load(c, ra, kb + set, k_bytes);
#pragma unroll
            for (int c = 0; c < NB; ++c)
                st.sb[set][c] = tb.load(c, rb, kb + set, k_bytes);
        }
    }

    // acc += the product of tile tc over its nk <= PD K-tiles, all of which are
    // in the staging sets already (prefetch with n = nk): each goes to its own
    // stage, one barrier, then the K-steps in order -- the same instructions on
    // the same fragments as the main loop.  The persistent kernel runs short K
    // this way, so that none of a tile's loads is issued after the previous
    // tile's D stores: a wait for such a load would also wait for those stores
    // to drain (one counter covers vector loads and stores, in order).
    template <bool PARK_IN_STAGES>
    static __device__ __forceinline__ void short_loop(const GemmParams &p, const TileCoord tc, int nk, char *smem,
                                                      acc_t (&acc)[MT][NT], uint32_t tid, Staging &st)
    {
        const uint32_t lane = tid & 63u;
        const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const uint32_t wm = wave / WGN, wn = wave % WGN;
        const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
        ATile ta;
        BTile tb;
        if constexpr (AMODE == MC16 || AMODE == MC8)
            ta.init(p.lda * E, p.M - m0, wave, lane);
        else
            ta.init(p.lda * E, wave, lane);
        if constexpr (BMODE == MC16 || BMODE == MC8)
            tb.init(p.ldb * E, p.N - n0, wave, lane);
        else
            tb.init(p.ldb * E, wave, lane);
        const uint32_t k_bytes = (uint32_t)p.K * E;
        if constexpr (AMODE == KCD)
            ta.init_mask(k_bytes);
        if constexpr (BMODE == KCD)
            tb.init_mask(k_bytes);
#pragma unroll
        for (int set = 0; set < PD; ++set) {
            if (set > 0 && set >= nk)
                break;
            char *stage = smem + set * STAGE;
#pragma unroll
            for (int c = 0; c < NA; ++c)
                ta.store(c, stage, wave, lane, st.sa[set][c], set, k_bytes);
#pragma unroll
            for (int c = 0; c < NB; ++c)
                tb.store(c, stage + ABYTES, wave, lane, st.sb[set][c], set, k_bytes);
        }
        stage_barrier();
        // B's fragments of a K-step, then A's one tile row at a time (registers: the
        // staging sets are still live beside the accumulators)
        u32x4 af[FH], bfr[NT][FH];
#pragma unroll
        for (int set = 0; set < PD; ++set) {
            if (set > 0 && set >= nk)
                break;
            const char *stage = smem + set * STAGE;
#pragma unroll
            for (int ks = 0; ks < (F8 ? 1 : 2); ++ks) {
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int h = 0; h < FH; ++h)
                        bfr[j][h] = BTile::frag(stage + ABYTES, wn * WTN + j * 16, F8 ? h : ks, lane);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
#pragma unroll
                    for (int h = 0; h < FH; ++h)
                        af[h] = ATile::frag(stage, wm * WTM + i * 16, F8 ? h : ks, lane);
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        if constexpr (F8)
                            acc[i][j] = Mfma<E4M3>::step2(bfr[j][0], bfr[j][1], af[0], af[1], acc[i][j]);
                        else
                            acc[i][j] = Mfma<T>::step(bfr[j][0], af[0], acc[i][j]);
                    }
                }
            }
        }
        // Every fragment read above came after the one barrier: an epilogue that
        // parks each wavefront's results in the stages must wait until all
        // wavefronts are done reading them (the main loop's reads after its last
        // barrier are of a K-tile past the range, whose values are never used).
        if constexpr (PARK_IN_STAGES)
            stage_barrier();
    }

    // acc += the product of tile tc over K-tiles [kb, ke) (kb < ke), with the
    // caller's staging registers st (PRE: K-tile kb is already in set 0, loaded
    // by prefetch).  smem holds two stages; K-tile kt uses stage kt mod 2.
    // tid is threadIdx.x (a caller that loops over tiles passes an opaque copy,
    // so that the lane arithmetic is not hoisted out of its loop and kept in
    // registers).
    template <bool PRE = false>
    static __device__ __forceinline__ void mainloop(const GemmParams &p, const TileCoord tc, int kb, int ke,
                                                    char *smem, acc_t (&acc)[MT][NT], uint32_t tid, Staging &st)
    {
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave / WGN, wn = wave % WGN;
    const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;

    // Each operand's descriptor starts at this tile's first row (K-contiguous)
    // or column (M/N-contiguous) and ends with the batch slice.
    const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
    const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;
    const int64_t a_start = (AMODE == MC16 || AMODE == MC8) ? m0 * E : m0 * p.lda * E;
    const int64_t b_start = (BMODE == MC16 || BMODE == MC8) ? n0 * E : n0 * p.ldb * E;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_start, (uint32_t)((p.a_bytes - a_start + 3) & ~3ll));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_start, (uint32_t)((p.b_bytes - b_start + 3) & ~3ll));

    ATile ta;
    BTile tb;
    if constexpr (AMODE == MC16 || AMODE == MC8)
        ta.init(p.lda * E, p.M - m0, wave, lane);
    else
        ta.init(p.lda * E, wave, lane);
    if constexpr (BMODE == MC16 || BMODE == MC8)
        tb.init(p.ldb * E, p.N - n0, wave, lane);
    else
        tb.init(p.ldb * E, wave, lane);
    const uint32_t k_bytes = (uint32_t)p.K * E;
    if constexpr (AMODE == KCD)
        ta.init_mask(k_bytes);
    if constexpr (BMODE == KCD)
        tb.init_mask(k_bytes);

    // K-tiles between their global loads and their LDS writes, PD sets
    auto &sa = st.sa;
    auto &sb = st.sb;
    auto load_one = [&](int c, int kt, int set = 0) {
        if (c < NA)
            sa[set][c] = ta.load(c, ra, kt, k_bytes);
        else
            sb[set][c - NA] = tb.load(c - NA, rb, kt, k_bytes);
    };
    auto store_one = [&](int c, char *stage, int kt, int set = 0) { // staging set holds K-tile kt
        if (c < NA)
            ta.store(c, stage, wave, lane, sa[set][c], kt, k_bytes);
        else
            tb.store(c - NA, stage + ABYTES, wave, lane, sb[set][c - NA], kt, k_bytes);
    };
    // the debug build's poison of this wavefront's slots of a retired stage
    auto poison = [&](char *stage) {
        if constexpr (DMU_LDS_POISON) {
            const u32x4 ones = {~0u, ~0u, ~0u, ~0u};
#pragma unroll
            for (int c = 0; c < NA; ++c)
                ta.store_raw(c, stage, wave, ones);
#pragma unroll
            for (int c = 0; c < NB; ++c)
                tb.store_raw(c, stage + ABYTES, wave, ones);
        }
    };

    // Operand fragments of one K-step (e4m3: both K-step halves of the K-tile,
    // which one MFMA consumes together).
    u32x4 af[MT][FH], bfr[NT][FH];
    auto read_a = [&](int i, const char *stage, int ks) {
#pragma unroll
        for (int h = 0; h < FH; ++h)
            af[i][h] = ATile::frag(stage, wm * WTM + i * 16, F8 ? h : ks, lane);
    };
    auto read_b = [&](int j, const char *stage, int ks) {
#pragma unroll
        for (int h = 0; h < FH; ++h)
            bfr[j][h] = BTile::frag(stage + ABYTES, wn * WTN + j * 16, F8 ? h : ks, lane);
    };
    // zero: std::true_type for the first K-step of the range on AGPR
    // accumulators (the product starts from a zero accumulator operand)
    auto mfma = [&](int i, int j, auto zero) {
        if constexpr (F8)
            acc[i][j] = Mfma<E4M3>::step2(bfr[j][0], bfr[j][1], af[i][0], af[i][1], acc[i][j]);
        else if constexpr (AG && decltype(zero)::value)
            Mfma<T>::step_a0(bfr[j][0], af[i][0], acc[i][j]);
        else if constexpr (AG)
            Mfma<T>::step_a(bfr[j][0], af[i][0], acc[i][j]);
        else
            acc[i][j] = Mfma<T>::step(bfr[j][0], af[i][0], acc[i][j]);
    };
    const std::false_type acc_in{};

    constexpr int NLD = NA + NB;

    {
        // with two staging sets the stages alternate from stage 0 at kb
        char *first = PD == 2 ? smem : smem + (kb & 1) * STAGE;
        if constexpr (!PRE) {
#pragma unroll
            for (int c = 0; c < NLD; ++c)
                load_one(c, kb);
        }
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            store_one(c, first, kb);
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            load_one(c, kb + 1, PD - 1);
        if constexpr (PD == 2) {
#pragma unroll
            for (int c = 0; c < NLD; ++c)
                load_one(c, kb + 2, 0);
        }
        stage_barrier();
#pragma unroll
        for (int i = 0; i < MT; ++i)
            read_a(i, first, 0);
#pragma unroll
        for (int j = 0; j < NT; ++j)
            read_b(j, first, 0);
    }

    // MFMA order within a K-step: two halves of the tile rows, each walked
    // column by column -- slot q is tile (row_of(q), col_of(q)).  Every fragment
    // is reloaded right after its last use; the order leaves at least
    // min(MN/2 + MT/2, MN/2 - MT/2 + 1) MFMAs between a reload and the next use.
    constexpr int HM = MT / 2, HALF = MN / 2;
    auto row_of = [](int q) { return (q / HALF) * HM + (q % HALF) % HM; };
    auto col_of = [](int q) { return (q % HALF) / HM; };
    auto last_a = [](int i) { return (i / HM) * HALF + (NT - 1) * HM + i % HM; }; // slot of A_i's last use
    auto last_b = [](int j) { return HALF + j * HM + HM - 1; };                  // slot of B_j's last use

    // Staging copies (K-tile kt+1 to the free stage, then the loads of K-tile
    // kt+2 into the same registers) ride on the MFMAs of K-step 0 and of the
    // first half of K-step 1, ahead of the stage hand-over.  K-tiles past K
    // read as zeros through the range check, so the body is branch-free.
    constexpr int SLOTS = MN + HALF;
    if constexpr (F8) {
        // e4m3: one K-step per K-tile.  First half: the staging copies; the
        // barrier; second half: each fragment of K-tile kt+1 is read from the
        // other stage right after its last use (the first half's A rows at
        // once).  Every read of a stage happens before the barrier that
        // precedes its overwrite.
        auto ktile8 = [&](int kt, char *nxt, int set) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < HALF; ++q) {
                mfma(row_of(q), col_of(q), acc_in);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ci = q * NLD / HALF; ci < (q + 1) * NLD / HALF; ++ci) {
                    store_one(ci, nxt, kt + 1, set);
                    load_one(ci, kt + 1 + PD, set);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            stage_barrier();
            poison(nxt == smem ? smem + STAGE : smem); // K-tile kt's stage: read no more
#pragma unroll
            for (int q = HALF; q < MN; ++q) {
                const int i = row_of(q), j = col_of(q), h = q - HALF;
                mfma(i, j, acc_in);
                __builtin_amdgcn_sched_barrier(0);
                if (h < HM)
                    read_a(h, nxt, 0);
                if (q == last_b(j))
                    read_b(j, nxt, 0);
                if (q == last_a(i))
                    read_a(i, nxt, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if constexpr (PD == 2) {
            int kt = kb;
            for (; kt + 1 < ke; kt += 2) {
                ktile8(kt, smem + STAGE, 1);
                ktile8(kt + 1, smem, 0);
            }
            if (kt < ke)
                ktile8(kt, smem + STAGE, 1);
        } else {
            for (int kt = kb; kt < ke; ++kt)
                ktile8(kt, smem + ((kt + 1) & 1) * STAGE, 0);
        }
    } else {
    // One K-tile: K-tile kt is in stage cur, K-tile kt+1 goes from staging
    // set `set` to stage nxt, and K-tile kt+1+PD is loaded into that set.
    // zero: std::true_type for the range's first K-tile on AGPR accumulators.
    auto ktile = [&](auto zero, int kt, char *cur, char *nxt, int set) __attribute__((always_inline)) {
        // K-step 0; each fragment of K-step 1 is read right after its last use.
#pragma unroll
        for (int q = 0; q < MN; ++q) {
            const int i = row_of(q), j = col_of(q);
            mfma(i, j, zero);
            __builtin_amdgcn_sched_barrier(0); // reads below reuse the registers this MFMA reads
            if (q == last_b(j))
                read_b(j, cur, 1);
            if (q == last_a(i))
                read_a(i, cur, 1);
#pragma unroll
            for (int ci = q * NLD / SLOTS; ci < (q + 1) * NLD / SLOTS; ++ci) {
                store_one(ci, nxt, kt + 1, set);
                load_one(ci, kt + 1 + PD, set);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // K-step 1, first half: the remaining staging copies.
#pragma unroll
        for (int q = 0; q < HALF; ++q) {
            const int i = row_of(q), j = col_of(q);
            mfma(i, j, acc_in);
            __builtin_amdgcn_sched_barrier(0);
            const int slot = MN + q;
#pragma unroll
            for (int ci = slot * NLD / SLOTS; ci < (slot + 1) * NLD / SLOTS; ++ci) {
                store_one(ci, nxt, kt + 1, set);
                load_one(ci, kt + 1 + PD, set);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_barrier();
        poison(cur); // K-tile kt's stage: its last fragment reads are done
        // Second half: K-step 0 of K-tile kt+1 from the other stage -- first the
        // A fragments of the rows already done, one per MFMA, then each
        // remaining fragment right after its last use.
#pragma unroll
        for (int q = HALF; q < MN; ++q) {
            const int i = row_of(q), j = col_of(q), h = q - HALF;
            mfma(i, j, acc_in);
            __builtin_amdgcn_sched_barrier(0);
            if (h < HM)
                read_a(h, nxt, 0);
            if (q == last_b(j))
                read_b(j, nxt, 0);
            if (q == last_a(i))
                read_a(i, nxt, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (AG) {
        // the first K-tile peeled: its K-step 0 writes the accumulators from zero
        static_assert(PD == 1, "one staging set on the four-wavefront tile");
        ktile(std::true_type{}, kb, smem + (kb & 1) * STAGE, smem + ((kb + 1) & 1) * STAGE, 0);
        for (int kt = kb + 1; kt < ke; ++kt)
            ktile(acc_in, kt, smem + (kt & 1) * STAGE, smem + ((kt + 1) & 1) * STAGE, 0);
    } else if constexpr (PD == 2) {
        // two K-tiles per iteration: the staging set and both stages are
        // fixed for each of them
        int kt = kb;
        for (; kt + 1 < ke; kt += 2) {
            ktile(acc_in, kt, smem, smem + STAGE, 1);
            ktile(acc_in, kt + 1, smem + STAGE, smem, 0);
        }
        if (kt < ke)
            ktile(acc_in, kt, smem, smem + STAGE, 1);
    } else {
        for (int kt = kb; kt < ke; ++kt)
            ktile(acc_in, kt, smem + (kt & 1) * STAGE, smem + ((kt + 1) & 1) * STAGE, 0);
    }
    }
    if constexpr (AG) {
        // The MFMAs above are assembly the compiler does not see as matrix
        // instructions, so it cannot space the first reads of their results
        // (v_accvgpr_read in the epilogue) from the last writes: 32 wait states
        // here, after every MFMA (all are volatile, as is this), and the
        // accumulators pass through empty volatile statements after it, so no
        // read of them moves above the wait.
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                asm volatile("" : "+a"(acc[i][j]));
    }
    }

    // D = epilogue(acc) for tile tc.  Every wavefront must be past the last
    // barrier of the main loop and read no stage any more: each parks its
    // results in its own part of the stages.
    static __device__ __forceinline__ void epilogue(const GemmParams &p, const TileCoord te, const acc_t (&acc)[MT][NT],
                                                    char *smem, uint32_t lane, uint32_t wave)
    {
        const char *Cb = p.C ? p.C + (int64_t)te.b * p.stride_c * dt_bytes(O) : nullptr;
        char *Db = p.D + (int64_t)te.b * p.stride_d * dt_bytes(O);
        store_staged<O, MT, NT>(p, acc, smem + wave * PARK, (int64_t)te.tm * BM + (wave / WGN) * WTM,
                                (int64_t)te.tn * BN + (wave % WGN) * WTN, lane, Cb, Db, epi_ptrs(p, te.b));
    }

    // One tile's accumulators to / from a partial-sum slot of PARTIAL_BYTES:
    // (wavefront, tile i, tile j) blocks of 64 lanes x 16 bytes, coalesced.
    // The accesses are coherent at device scope (cache policy SC1): stores are
    // written through to the coherence point and loads do not hit a stale copy
    // in this XCD's L2 or this unit's L1, so that no cache-wide write-back or
    // invalidation is needed around the exchange.
    static constexpr int SC1 = 16; // cache-policy bit of the buffer instructions
    static __device__ __forceinline__ void store_partial(char *slot, const acc_t (&acc)[MT][NT], uint32_t lane,
                                                         uint32_t wave)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(slot, PARTIAL_BYTES);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), r, lane * 16,
                                                       ((wave * MT + i) * NT + j) * 1024, SC1);
    }
    // A whole slot into registers: every load is issued before any is used, since
    // each round trip to the coherence point costs about a microsecond.
    static __device__ __forceinline__ void load_partial(const char *slot, acc_t (&v)[MT][NT], uint32_t lane,
                                                        uint32_t wave)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(slot, PARTIAL_BYTES);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                v[i][j] = __builtin_bit_cast(acc_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        r, lane * 16, ((wave * MT + i) * NT + j) * 1024, SC1));
    }
    static __device__ __forceinline__ void add_into(acc_t (&acc)[MT][NT], const acc_t (&v)[MT][NT])
    {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[i][j] += v[i][j];
    }
};

// Eight wavefronts run two per SIMD, four one per SIMD (with the AGPRs).
template <int T, int O, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
    __attribute__((amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4))) gemm_tiled(GemmParams p)
{
    typedef Tiled<T, O, BM, BN, WGM, WGN, AMODE, BMODE> G;
    __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE];
    typename G::acc_t acc[G::MT][G::NT];
    const int nk = (int)(((int64_t)p.K * G::E + 127) / 128);
    phase_begin(p.phases, blockIdx.x, (uint32_t)nk);
    if constexpr (!G::AG) {
#pragma unroll
        for (int i = 0; i < G::MT; ++i)
#pragma unroll
            for (int j = 0; j < G::NT; ++j)
                acc[i][j] = typename G::acc_t{};
    }
    if (nk > 0) {
        typename G::Staging st;
        G::mainloop(p, tile_of(p, blockIdx.x), 0, nk, smem, acc, threadIdx.x, st);
    } else if constexpr (G::AG) {
        // K == 0: D = C (the main loop writes the accumulators otherwise)
#pragma unroll
        for (int i = 0; i < G::MT; ++i)
#pragma unroll
            for (int j = 0; j < G::NT; ++j)
                acc[i][j] = typename G::acc_t{};
    }
    // The tile coordinates and lane are derived afresh from opaque copies of
    // the ids, so that the compiler does not keep the values of the prologue
    // alive (in registers the loop needs) across the K loop.
    uint32_t wg2 = blockIdx.x, tid2 = threadIdx.x;
    asm volatile("" : "+s"(wg2));
    asm volatile("" : "+v"(tid2));
    phase_mark(p.phases, wg2, PH_LOOP);
    phase_mark(p.phases, wg2, PH_FIX);
    G::epilogue(p, tile_of(p, wg2), acc, smem, tid2 & 63u, __builtin_amdgcn_readfirstlane(tid2 >> 6));
    phase_end(p.phases, wg2);
}


// The persistent form of the tiled kernel ("Tensor Cores, CUTLASS and CuTe"
// section 6.5: a fixed number of blocks looping over the output tiles): W
// workgroups, one per compute unit, take the tiles of the one-per-tile launch
// in turn (virtual workgroup ids w, w + W, ..., which keep each worker on its
// XCD when W is a multiple of 8).  Before a tile's epilogue, the worker loads
// the first K-tile of its next tile into the staging registers, so that those
// loads are in flight while D is written, and no workgroup launch separates
// the tiles.  Same main loop and epilogue: bit-identical to gemm_tiled.
template <int T, int O, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
    __attribute__((amdgpu_waves_per_eu(2, 2))) gemm_persist(GemmParams p)
{
    typedef Tiled<T, O, BM, BN, WGM, WGN, AMODE, BMODE> G;
    // K of at most PD K-tiles: each tile's whole K range is loaded before the
    // previous tile's epilogue (short_loop; not on the 256 x 256 tile, whose one
    // staging set leaves no registers for it, nor for e4m3, whose fragments are
    // twice as large: both spilled).  Those configurations park the epilogue's
    // results beside the stages (LDS: 256 x 128, 96 + 35 KiB), so that a
    // wavefront done with its K-steps parks while others still read the stages.
    constexpr bool SHORT = G::PD >= 2 && !G::F8;
    __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE + (SHORT ? G::NW * G::PARK : 0)];
    typename G::Staging st;
    const uint32_t W = gridDim.x, total = p.total_tiles;
    const int nk = (int)(((int64_t)p.K * G::E + 127) / 128);
    uint32_t t = blockIdx.x;
    if (t >= total)
        return; // more workers than tiles (uniform: before any barrier)
    const bool short_k = SHORT && nk <= G::PD;
    if (nk > 0)
        G::prefetch(p, tile_of(p, t), 0, st, threadIdx.x, short_k ? nk : 1);
    for (; t < total; t += W) {
        phase_begin(p.phases, t, (uint32_t)nk);
        typename G::acc_t acc[G::MT][G::NT];
#pragma unroll
        for (int i = 0; i < G::MT; ++i)
#pragma unroll
            for (int j = 0; j < G::NT; ++j)
                acc[i][j] = typename G::acc_t{};
        uint32_t tid_m = threadIdx.x;
        asm volatile("" : "+v"(tid_m));
        if constexpr (SHORT) {
            if (nk > 0 && short_k)
                G::template short_loop<false>(p, tile_of(p, t), nk, smem, acc, tid_m, st);
            else if (nk > 0)
                G::template mainloop<true>(p, tile_of(p, t), 0, nk, smem, acc, tid_m, st);
        } else if (nk > 0) {
            G::template mainloop<true>(p, tile_of(p, t), 0, nk, smem, acc, tid_m, st);
        }
        uint32_t tid_e = threadIdx.x, t2 = t;
        asm volatile("" : "+v"(tid_e));
        asm volatile("" : "+s"(t2));
        phase_mark(p.phases, t2, PH_LOOP);
        if (nk > 0 && t2 + W < total)
            G::prefetch(p, tile_of(p, t2 + W), 0, st, tid_e, short_k ? nk : 1);
        phase_mark(p.phases, t2, PH_FIX);
        G::epilogue(p, tile_of(p, t2), acc, (SHORT && short_k) ? smem + 2 * G::STAGE : smem, tid_e & 63u,
                    __builtin_amdgcn_readfirstlane(tid_e >> 6));
        phase_end(p.phases, t2);
        __syncthreads(); // every wavefront is done with its park before the next tile's stages
    }
}

} // namespace dmu
