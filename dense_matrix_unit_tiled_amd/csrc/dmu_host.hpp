// Host-side helpers of the C ABI: thread-local error text, launch checks and
// the per-type launcher entry points implemented in dmu_launch_*.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dmu_device.hpp"

namespace dmu {

void set_error(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// Phase log (dmu_phase_log): when a log is set, checks that it holds `records`
// records and points *log at it (else leaves *log NULL), and remembers the
// launch's record count and `kind` for dmu_phase_log_last.  DMU_ERR_INVALID_ARG
// (message set) when the log is too small.
int phase_reserve(size_t records, int kind, const char *who, uint64_t **log);
// DMU_OK, or DMU_ERR_HIP with the runtime's message when the last launch failed.
int check_launch(const char *what);

// Kernel shapes of the tiled kernel (gemm_tiled, 8 wavefronts) and the
// fallback (gemm_generic).
enum TileCfg {
    TILE_256x256 = 0,   // wavefronts 2 x 4, 128 x 64 each
    TILE_256x128 = 1,   // wavefronts 4 x 2, 64 x 64 each
    TILE_128x128 = 2,   // wavefronts 2 x 4, 64 x 32 each
    TILE_GENERIC = 3,   // 64 x 64, element loads
    TILE_256x256W4 = 4, // wavefronts 2 x 2, 128 x 128 each, accumulators in AGPRs (16-bit and int8 inputs)
    TILE_64x128 = 5,    // wavefronts 2 x 4, 32 x 32 each (A K-contiguous; data-parallel only)
    NUM_TILE_CFGS = 6
};

struct LaunchCfg {
    int tile;    // TileCfg
    int amode;   // Mode of A (ignored for TILE_GENERIC)
    int bmode;   // Mode of B
    int workers; // > 0: the persistent form of the tiled kernel on this many workgroups
};

inline int tile_bm(int tile)
{
    return (tile == TILE_GENERIC || tile == TILE_64x128) ? 64 : (tile == TILE_128x128 ? 128 : 256);
}
inline int tile_bn(int tile)
{
    return tile == TILE_GENERIC ? 64 : ((tile == TILE_256x256 || tile == TILE_256x256W4) ? 256 : 128);
}

// One launcher per (input type, output type); each returns hipSuccess or the
// launch error.  The grid is p.total_tiles workgroups.
hipError_t launch_f16_f32(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_f16_f16(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_bf16_bf16(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_bf16_f32(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_i8_i32(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_i8_f32(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_i8_f16(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_i8_bf16(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_e4m3_f32(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_e4m3_f16(const LaunchCfg &c, const GemmParams &p, hipStream_t s);
hipError_t launch_e4m3_bf16(const LaunchCfg &c, const GemmParams &p, hipStream_t s);

// The stream-K launchers (tiled configurations only; grid = sk.workers).
#define DMU_DECLARE_SK(name) \
    hipError_t name##_sk(const LaunchCfg &c, const GemmParams &p, const StreamKParams &sk, hipStream_t s);
DMU_DECLARE_SK(launch_f16_f32)
DMU_DECLARE_SK(launch_f16_f16)
DMU_DECLARE_SK(launch_bf16_bf16)
DMU_DECLARE_SK(launch_bf16_f32)
DMU_DECLARE_SK(launch_i8_i32)
DMU_DECLARE_SK(launch_i8_f32)
DMU_DECLARE_SK(launch_i8_f16)
DMU_DECLARE_SK(launch_i8_bf16)
DMU_DECLARE_SK(launch_e4m3_f32)
DMU_DECLARE_SK(launch_e4m3_f16)
DMU_DECLARE_SK(launch_e4m3_bf16)
#undef DMU_DECLARE_SK

} // namespace dmu
