// Single-wavefront layout probes: the gfx950 counterpart of the isolated
// layout experiment (KingOfEgg, sections 6-7), which checks one matrix
// instruction and its fragment loads lane by lane and register by register
// before they are used in a large kernel.
#include <hip/hip_runtime.h>

#include "../../include/dmu.h"
#include "dmu_host.hpp"
#include "dmu_tiled.hpp"

namespace dmu {

// Operand fragment of an m x k (row-major, in_type) matrix X for lane l:
// row l % m, the 16 bytes starting at byte 16 * (l / m) of that row.
__device__ __forceinline__ u32x4 probe_frag(const char *x, int m, int row_bytes, uint32_t lane)
{
    const uint32_t row = lane % (uint32_t)m, part = lane / (uint32_t)m;
    return *reinterpret_cast<const u32x4 *>(x + row * row_bytes + part * 16);
}

template <int V>
__global__ void __launch_bounds__(64) probe_mfma(const char *a, const char *bt, uint32_t *out)
{
    const uint32_t l = threadIdx.x;
    if (V == DMU_PROBE_MFMA_32x32x16_BF16 || V == DMU_PROBE_MFMA_32x32x16_F16) {
        const u32x4 x = probe_frag(a, 32, 32, l), y = probe_frag(bt, 32, 32, l);
        f32x16 c = {};
        if (V == DMU_PROBE_MFMA_32x32x16_BF16)
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                        c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c,
                                                       0, 0, 0);
        for (int r = 0; r < 16; ++r) {
            const float v = c[r]; // copy the element out first: a bit_cast of a vector element lvalue mis-lowers
            out[l * 16 + r] = __builtin_bit_cast(uint32_t, v);
        }
    } else if (V == DMU_PROBE_MFMA_16x16x32_BF16 || V == DMU_PROBE_MFMA_16x16x32_F16) {
        const u32x4 x = probe_frag(a, 16, 64, l), y = probe_frag(bt, 16, 64, l);
        f32x4 c = {};
        if (V == DMU_PROBE_MFMA_16x16x32_BF16)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                        c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c,
                                                       0, 0, 0);
        for (int r = 0; r < 4; ++r) {
            const float v = c[r];
            out[l * 4 + r] = __builtin_bit_cast(uint32_t, v);
        }
    } else if (V == DMU_PROBE_MFMA_32x32x32_I8) {
        const u32x4 x = probe_frag(a, 32, 32, l), y = probe_frag(bt, 32, 32, l);
        i32x16 c = {};
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, x), __builtin_bit_cast(i32x4, y), c, 0, 0,
                                                  0);
        for (int r = 0; r < 16; ++r)
            out[l * 16 + r] = (uint32_t)c[r];
    } else if (V == DMU_PROBE_MFMA_16x16x128_E4M3) {
        // the GEMM kernels' two 16-byte fragments of a 128-byte row: bytes
        // 16 (l / 16) .. +15 and 64 + 16 (l / 16) .. +15 of row l % 16
        const u32x4 x0 = probe_frag(a, 16, 128, l), x1 = probe_frag(a + 64, 16, 128, l);
        const u32x4 y0 = probe_frag(bt, 16, 128, l), y1 = probe_frag(bt + 64, 16, 128, l);
        const f32x4 c = Mfma<E4M3>::step2(x0, x1, y0, y1, f32x4{});
        for (int r = 0; r < 4; ++r) {
            const float v = c[r];
            out[l * 4 + r] = __builtin_bit_cast(uint32_t, v);
        }
    } else if (V == DMU_PROBE_MFMA_16x16x64_I8) {
        const u32x4 x = probe_frag(a, 16, 64, l), y = probe_frag(bt, 16, 64, l);
        i32x4 c = {};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, x), __builtin_bit_cast(i32x4, y), c, 0, 0,
                                                  0);
        for (int r = 0; r < 4; ++r)
            out[l * 4 + r] = (uint32_t)c[r];
    }
}

// v_permlane16_swap / v_permlane32_swap with both operands equal: lane l writes
// the two results of each.
__global__ void __launch_bounds__(64) probe_lane_swap(const uint32_t *in, uint32_t *out)
{
    const uint32_t l = threadIdx.x, v = in[l];
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const uint32_t a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
    out[4 * l + 0] = a0;
    out[4 * l + 1] = a1;
    out[4 * l + 2] = b0;
    out[4 * l + 3] = b1;
}

// LDS image of 4096 bytes: each of the 64 lanes copies 64 bytes.
__device__ __forceinline__ void probe_fill_lds(char *lds, const char *img, uint32_t l)
{
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4 *>(lds + l * 64 + q * 16) = *reinterpret_cast<const u32x4 *>(img + l * 64 + q * 16);
}

__global__ void __launch_bounds__(64) probe_lds_b128(const char *img, const int32_t *addr, uint32_t *out)
{
    __shared__ __attribute__((aligned(16))) char lds[4096];
    const uint32_t l = threadIdx.x;
    probe_fill_lds(lds, img, l);
    __syncthreads();
    const uint32_t off = (uint32_t)addr[l] & (4096u - 16u); // aligned and in bounds
    const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + off);
    for (int e = 0; e < 4; ++e)
        out[l * 4 + e] = v[e];
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(64) probe_lds_tr16(const char *img, const int32_t *addr, uint32_t *out)
{
    __shared__ __attribute__((aligned(16))) char lds[4096];
    const uint32_t l = threadIdx.x;
    probe_fill_lds(lds, img, l);
    __syncthreads();
    const uint32_t off = (uint32_t)addr[l] & (4096u - 8u); // aligned and in bounds
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(lds + off));
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    out[l * 2 + 0] = w[0];
    out[l * 2 + 1] = w[1];
}

// ds_read_b64_tr_b8: lane l reads at addr[l] (aligned to 8 bytes, in bounds).
typedef int i32x2 __attribute__((ext_vector_type(2)));
__global__ void __launch_bounds__(64) probe_lds_tr8(const char *img, const int32_t *addr, uint32_t *out)
{
    __shared__ __attribute__((aligned(16))) char lds[4096];
    const uint32_t l = threadIdx.x;
    probe_fill_lds(lds, img, l);
    __syncthreads();
    const uint32_t off = (uint32_t)addr[l] & (4096u - 8u);
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(lds + off));
    out[l * 2 + 0] = (uint32_t)v[0];
    out[l * 2 + 1] = (uint32_t)v[1];
}

// The tiled kernel's K-contiguous LDS format: a 32-row x 128-byte tile is
// written with the kernel's staging writes (transfer q, lane l carrying row
// 8q + l/8, chunk l%8) and read back with its fragment reads for row blocks 0
// and 16, K-steps 0 and 1.
// Output per lane: [row block][K-step][16 bytes].
__global__ void __launch_bounds__(64) probe_lds_frag(const char *tile, uint32_t *out)
{
    typedef KcTile<32, 1, false> Tile;
    __shared__ __attribute__((aligned(1024))) char lds[Tile::BYTES];
    const uint32_t l = threadIdx.x;
    for (int q = 0; q < Tile::NL; ++q) {
        const uint32_t row = 8 * q + l / 8, chunk = l % 8;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(tile + row * 128u + chunk * 16u);
        Tile t;
        t.init(128, 0, l);
        t.store(q, lds, 0, l, v, 0, 128);
    }
    __syncthreads();
    for (int rb = 0; rb < 2; ++rb)
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 v = Tile::frag(lds, 16 * rb, ks, l);
            for (int e = 0; e < 4; ++e)
                out[((l * 2 + rb) * 2 + ks) * 4 + e] = v[e];
        }
}

// The tiled kernel's M/N-contiguous 16-bit LDS format: a 64 K-row x 128-value
// tile (row-major, 256 bytes per K-row) is written with the kernel's staging
// writes of all eight wavefronts' transfers and read back with its transposing
// fragment reads for column blocks 0, 16, .., 112 and K-steps 0 and 1.
// Output per lane: [column block][K-step][8 16-bit values].
__global__ void __launch_bounds__(64) probe_lds_frag_t(const char *tile, uint32_t *out)
{
    typedef McTile<128, 8> Tile;
    __shared__ __attribute__((aligned(1024))) char lds[Tile::BYTES];
    const uint32_t l = threadIdx.x;
    for (uint32_t w = 0; w < 8; ++w) {
        Tile t;
        t.init(256, 128, w, l);
        for (int i = 0; i < Tile::NL; ++i) {
            const uint32_t k = (w * Tile::NL + i) * Tile::RPI + l / Tile::CPR, chunk = l % Tile::CPR;
            t.store(i, lds, w, l, *reinterpret_cast<const u32x4 *>(tile + k * 256u + chunk * 16u), 0, 0);
        }
    }
    __syncthreads();
    for (int cb = 0; cb < 8; ++cb)
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 v = Tile::frag(lds, 16 * cb, ks, l);
            for (int e = 0; e < 4; ++e)
                out[((l * 8 + cb) * 2 + ks) * 4 + e] = v[e];
        }
}

template <int O>
__global__ void __launch_bounds__(64) probe_cvt(const float *in, uint16_t *out)
{
    const uint32_t l = threadIdx.x;
    for (int q = 0; q < 4; ++q) {
        const auto h = Out<O>::from_acc(in[l * 4 + q]);
        out[l * 4 + q] = __builtin_bit_cast(uint16_t, h);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core ceiling (diagnostics): the rate this chip sustains for the GEMM
// kernels' 16 x 16 instructions when nothing else runs.  A grid shaped like the
// 4096^3 launch (workgroups of 8 wavefronts, two per SIMD) where every
// wavefront issues `rounds` x 32 independent MFMAs into 32 accumulators, the
// operands drawn from 4 x 4 register fragments of fixed pseudo-random finite
// values (data as varied as a real product's, so the power drawn is alike),
// with no memory traffic.  Thread 0 of each workgroup stamps the 100 MHz clock
// and the shader clock counter at start and end (4 words per workgroup).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    return x ^ (x >> 16);
}

template <int T>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
    mfma_ceiling(uint64_t *stamps, int rounds)
{
    typedef typename Mfma<T>::acc_t acc_t;
    const uint32_t l = threadIdx.x;
    // 16-bit inputs: sign and mantissa random, exponent fixed (finite values of
    // magnitude 1-2 in fp16, small in bf16); int8: any bits
    const uint32_t keep = T == I8 ? 0xffffffffu : 0x83ff83ffu, set = T == I8 ? 0u : 0x3c003c00u;
    u32x4 x[4], y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[i][e] = (mix32(l * 64 + i * 4 + e + 1) & keep) | set;
            y[i][e] = (mix32(l * 64 + i * 4 + e + 0x9e3779b9u) & keep) | set;
        }
    if (stamps != nullptr && l == 0) {
        stamps[blockIdx.x * 4 + 0] = __builtin_amdgcn_s_memrealtime();
        stamps[blockIdx.x * 4 + 1] = __builtin_amdgcn_s_memtime();
    }
    acc_t acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j)
        acc[j] = acc_t{};
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int j = 0; j < 32; ++j)
            acc[j] = Mfma<T>::step(x[j & 3], y[(j >> 2) & 3], acc[j]);
    }
    // the results stay live (no store: an empty statement that reads them)
#pragma unroll
    for (int j = 0; j < 32; ++j)
        asm volatile("" : : "v"(acc[j]));
    if (stamps != nullptr && l == 0) {
        stamps[blockIdx.x * 4 + 2] = __builtin_amdgcn_s_memrealtime();
        stamps[blockIdx.x * 4 + 3] = __builtin_amdgcn_s_memtime();
    }
}

} // namespace dmu

using namespace dmu;

extern "C" int dmu_mfma_ceiling(int in_type, int rounds, int workgroups, void *stamps, void *stream)
{
    clear_error();
    if (rounds < 1 || workgroups < 1) {
        set_error("dmu_mfma_ceiling: rounds and workgroups must be positive");
        return DMU_ERR_INVALID_ARG;
    }
    if ((uintptr_t)stamps % 8) {
        set_error("dmu_mfma_ceiling: stamps is not 8-byte aligned");
        return DMU_ERR_INVALID_ARG;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint64_t *st = static_cast<uint64_t *>(stamps);
    switch (in_type) {
    case DMU_BF16: hipLaunchKernelGGL(mfma_ceiling<BF16>, dim3(workgroups), dim3(512), 0, s, st, rounds); break;
    case DMU_F16: hipLaunchKernelGGL(mfma_ceiling<F16>, dim3(workgroups), dim3(512), 0, s, st, rounds); break;
    case DMU_I8: hipLaunchKernelGGL(mfma_ceiling<I8>, dim3(workgroups), dim3(512), 0, s, st, rounds); break;
    default:
        set_error("dmu_mfma_ceiling: input type %d has no ceiling kernel (bf16, fp16, int8)", in_type);
        return DMU_ERR_UNSUPPORTED;
    }
    return check_launch("dmu_mfma_ceiling");
}

extern "C" int dmu_probe_info(int variant, int *m, int *n, int *k, int *in_type, int *regs)
{
    int mm = 0, nn = 0, kk = 0, t = 0, r = 0;
    switch (variant) {
    case DMU_PROBE_MFMA_32x32x16_BF16: mm = 32, nn = 32, kk = 16, t = DMU_BF16, r = 16; break;
    case DMU_PROBE_MFMA_32x32x16_F16: mm = 32, nn = 32, kk = 16, t = DMU_F16, r = 16; break;
    case DMU_PROBE_MFMA_16x16x32_BF16: mm = 16, nn = 16, kk = 32, t = DMU_BF16, r = 4; break;
    case DMU_PROBE_MFMA_16x16x32_F16: mm = 16, nn = 16, kk = 32, t = DMU_F16, r = 4; break;
    case DMU_PROBE_MFMA_32x32x32_I8: mm = 32, nn = 32, kk = 32, t = DMU_I8, r = 16; break;
    case DMU_PROBE_MFMA_16x16x64_I8: mm = 16, nn = 16, kk = 64, t = DMU_I8, r = 4; break;
    case DMU_PROBE_MFMA_16x16x128_E4M3: mm = 16, nn = 16, kk = 128, t = DMU_E4M3, r = 4; break;
    case DMU_PROBE_LDS_READ_B128: r = 4; break;
    case DMU_PROBE_LDS_READ_TR16: r = 2; break;
    case DMU_PROBE_LDS_READ_TR8: r = 2; break;
    case DMU_PROBE_LDS_FRAG: r = 16; break;
    case DMU_PROBE_LDS_FRAG_T: r = 64; break;
    case DMU_PROBE_LANE_SWAP: t = DMU_I32, r = 4; break;
    case DMU_PROBE_CVT_BF16: t = DMU_F32, r = 2; break; /* 4 halves per lane */
    case DMU_PROBE_CVT_F16: t = DMU_F32, r = 2; break;
    default:
        set_error("dmu_probe_info: unknown probe variant %d", variant);
        return DMU_ERR_UNSUPPORTED;
    }
    if (m) *m = mm;
    if (n) *n = nn;
    if (k) *k = kk;
    if (in_type) *in_type = t;
    if (regs) *regs = r;
    return DMU_OK;
}

extern "C" int dmu_probe(int variant, const void *in0, const void *in1, void *out, void *stream)
{
    clear_error();
    int rc = dmu_probe_info(variant, nullptr, nullptr, nullptr, nullptr, nullptr);
    if (rc != DMU_OK)
        return rc;
    const bool needs_in1 = variant <= DMU_PROBE_LDS_READ_TR16 || variant == DMU_PROBE_LDS_READ_TR8;
    if (!in0 || !out || (needs_in1 && !in1)) {
        set_error("dmu_probe: null pointer");
        return DMU_ERR_INVALID_ARG;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char *a = static_cast<const char *>(in0), *b = static_cast<const char *>(in1);
    uint32_t *o = static_cast<uint32_t *>(out);
    switch (variant) {
#define DMU_PROBE_MFMA_CASE(V) \
    case V: hipLaunchKernelGGL(probe_mfma<V>, dim3(1), dim3(64), 0, s, a, b, o); break;
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_32x32x16_BF16)
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_32x32x16_F16)
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_16x16x32_BF16)
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_16x16x32_F16)
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_32x32x32_I8)
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_16x16x64_I8)
        DMU_PROBE_MFMA_CASE(DMU_PROBE_MFMA_16x16x128_E4M3)
#undef DMU_PROBE_MFMA_CASE
    case DMU_PROBE_LDS_READ_B128:
        hipLaunchKernelGGL(probe_lds_b128, dim3(1), dim3(64), 0, s, a, reinterpret_cast<const int32_t *>(b), o);
        break;
    case DMU_PROBE_LDS_READ_TR16:
        hipLaunchKernelGGL(probe_lds_tr16, dim3(1), dim3(64), 0, s, a, reinterpret_cast<const int32_t *>(b), o);
        break;
    case DMU_PROBE_LDS_READ_TR8:
        hipLaunchKernelGGL(probe_lds_tr8, dim3(1), dim3(64), 0, s, a, reinterpret_cast<const int32_t *>(b), o);
        break;
    case DMU_PROBE_LDS_FRAG: hipLaunchKernelGGL(probe_lds_frag, dim3(1), dim3(64), 0, s, a, o); break;
    case DMU_PROBE_LDS_FRAG_T: hipLaunchKernelGGL(probe_lds_frag_t, dim3(1), dim3(64), 0, s, a, o); break;
    case DMU_PROBE_LANE_SWAP:
        hipLaunchKernelGGL(probe_lane_swap, dim3(1), dim3(64), 0, s, reinterpret_cast<const uint32_t *>(a), o);
        break;
    case DMU_PROBE_CVT_BF16:
        hipLaunchKernelGGL(probe_cvt<BF16>, dim3(1), dim3(64), 0, s, reinterpret_cast<const float *>(a),
                           reinterpret_cast<uint16_t *>(o));
        break;
    case DMU_PROBE_CVT_F16:
        hipLaunchKernelGGL(probe_cvt<F16>, dim3(1), dim3(64), 0, s, reinterpret_cast<const float *>(a),
                           reinterpret_cast<uint16_t *>(o));
        break;
    }
    return check_launch("dmu_probe");
}
