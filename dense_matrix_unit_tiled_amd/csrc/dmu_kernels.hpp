// Fallback GEMM kernel for gfx950: D = A*B + C for operands whose alignment
// rules out the vector loads of the tiled kernel (dmu_tiled.hpp).
//
//  gemm_generic  64 x 64 tiles, element-by-element loads, one LDS buffer with
//              two barriers per K-tile (the simplest correct form, as in the
//              "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough).  Every
//              output element goes through the same sequence of 16 x 16 x 32
//              (int8: x 64; e4m3: one x 128 per K-tile) matrix instructions
//              over the same K-steps as in the tiled kernel, so the two give
//              bit-identical results on the same inputs.
#pragma once

#include "dmu_tiled.hpp"

namespace dmu {

template <int T> struct In;
template <> struct In<F16> { static constexpr int bytes = 2; };
template <> struct In<BF16> { static constexpr int bytes = 2; };
template <> struct In<I8> { static constexpr int bytes = 1; };
template <> struct In<E4M3> { static constexpr int bytes = 1; };

template <int T, int E> struct Elem;
template <int T> struct Elem<T, 2> { typedef uint16_t t; };
template <int T> struct Elem<T, 1> { typedef uint8_t t; };

// One operand's 64 rows x 128 bytes of K-tile k0 into LDS, element by
// element, in the K-contiguous layout of the tiled kernel (chunks of row r
// permuted by XOR with r mod 8) so that its fragment reads apply.
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
        const uint32_t byte = ke * E;
        *reinterpret_cast<et *>(tile + row * 128u + (((byte >> 4) ^ (row & 7u)) << 4) + (byte & 15u)) = v;
    }
}

// 64 x 64 tile, wavefront w owns the 32 x 32 block (w / 2, w % 2): 2 x 2 tiles
// of 16 x 16, stored straight from the accumulators (lane l: row l % 16,
// columns 4 (l / 16) .. +3 of each tile) through the same fused epilogue,
// masked at the M/N edges.
template <int T, int O>
__global__ void __launch_bounds__(256) gemm_generic(GemmParams p)
{
    constexpr int E = In<T>::bytes;
    typedef typename Mfma<T>::acc_t acc_t;
    typedef KcTile<64, 8, false> Frag; // fragment reads of the K-contiguous layout
    typedef typename Out<O>::t ot;
    __shared__ __attribute__((aligned(1024))) char smem[128 * 128];

    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    const TileCoord tc = tile_of(p, blockIdx.x);
    const int64_t m0 = (int64_t)tc.tm * 64, n0 = (int64_t)tc.tn * 64;
    const char *Ab = p.A + (int64_t)tc.b * p.stride_a * E;
    const char *Bb = p.B + (int64_t)tc.b * p.stride_b * E;
    acc_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = acc_t{};
    const int nk = (int)(((int64_t)p.K * E + 127) / 128);
    for (int kt = 0; kt < nk; ++kt) {
        const int64_t k0 = (int64_t)kt * (128 / E);
        generic_fill<T>(smem, Ab, p.lda, p.a_kc != 0, m0, p.M, k0, p.K, tid);
        generic_fill<T>(smem + 64 * 128, Bb, p.ldb, p.b_kc != 0, n0, p.N, k0, p.K, tid);
        __syncthreads();
        if constexpr (T == E4M3) { // one MFMA over both K-step halves, as in the tiled kernel
            u32x4 af[2][2], bf[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    af[i][h] = Frag::frag(smem, wm * 32 + 16 * i, h, lane);
                    bf[i][h] = Frag::frag(smem + 64 * 128, wn * 32 + 16 * i, h, lane);
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = Mfma<E4M3>::step2(bf[j][0], bf[j][1], af[i][0], af[i][1], acc[i][j]);
        } else {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4 af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    af[i] = Frag::frag(smem, wm * 32 + 16 * i, ks, lane);
                    bf[i] = Frag::frag(smem + 64 * 128, wn * 32 + 16 * i, ks, lane);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = Mfma<T>::step(bf[j], af[i], acc[i][j]);
            }
        }
        __syncthreads();
    }
    const char *Cb = p.C ? p.C + (int64_t)tc.b * p.stride_c * dt_bytes(O) : nullptr;
    char *Db = p.D + (int64_t)tc.b * p.stride_d * dt_bytes(O);
    const EpiPtrs ep = epi_ptrs(p, tc.b);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t m = m0 + wm * 32 + 16 * i + (lane & 15u);
        if (m >= p.M)
            continue;
        const ot *Crow = Cb ? reinterpret_cast<const ot *>(Cb) + m * p.ldc : nullptr;
        ot *Drow = reinterpret_cast<ot *>(Db) + m * p.ldd;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 32 + 16 * j + 4 * (lane >> 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < p.N)
                    Drow[n + e] = epi_one<O>(p.epi, p.act, acc[i][j][e], ep.rs ? ep.rs[m] : 1.0f,
                                             ep.cs ? ep.cs[n + e] : 1.0f, ep.bias ? ep.bias[n + e] : 0.0f,
                                             Crow != nullptr, Crow ? Crow[n + e] : ot{});
        }
    }
}

} // namespace dmu
