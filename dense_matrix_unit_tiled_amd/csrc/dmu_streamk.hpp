// Stream-K scheduling of the tiled kernel (gemm_streamk).
//
// "Tensor Cores, CUTLASS and CuTe" section 6.5 describes the persistent tile
// scheduler (a fixed number of blocks per multiprocessor, each looping over
// tiles, instead of one block per tile), and section 4.5 counts the plain
// one-tile-per-block dispatch among the gaps of its kernel.  The data-parallel
// kernel here gives each workgroup one output tile, so a tile count that is
// not a multiple of the number of compute units leaves units idle in the last
// wave -- the 5000 x 3000 problem has 240 tiles of 256 x 256 for 256 units.
// This kernel is persistent and splits work in K as well ("stream-K"): a grid
// of W workgroups ("workers", one per compute unit) shares the
// I = tiles x K-tiles multiply-accumulate iterations evenly; worker w owns
// an equal share (q or q + 1) of consecutive iterations, i.e. the end of one
// tile, whole tiles, and the start of another (W <= I: no range is empty).
//
//   order      each worker walks its tiles in decreasing order, K forward
//              inside a tile.  A tile split between workers is then started
//              first by the lower workers (its leading K-tiles are the last
//              tile of their ranges) and finished last by the worker that holds
//              its final K-tile, which is its "finisher".
//   exchange   a non-finishing worker (at most one tile per worker) writes its
//              fp32/int32 accumulators to its own slot of the workspace with
//              device-coherent stores, waits for them to complete, then raises
//              its flag; the finisher polls the flags of the lower workers that
//              share its tile, adds their slots (device-coherent loads, issued
//              after the flag was seen) in increasing worker order (a fixed
//              order: the result is reproducible launch to launch), clears the
//              flags, and runs the epilogue.  No cache-wide write-back or
//              invalidation is involved: an agent-scope acquire fence would
//              invalidate the whole L2 of the XCD, the other workers' A and B
//              tiles included (measured: the 5000 x 3000 x 2050 product took
//              172 us that way against 73 us data-parallel).
//   progress   waits only go from a worker to lower-numbered workers, which
//              the hardware dispatches first on each XCD; with one workgroup
//              per compute unit all of them are resident anyway.  Each wait is
//              bounded: past the limit the worker records an error word in the
//              workspace and goes on, so every wavefront always exits (the
//              result is then wrong, and the host query of the error word,
//              dmu_gemm_streamk_error, reports it).
#pragma once

#include "dmu_tiled.hpp"

namespace dmu {

// Worker w's range is [start(w), start(w + 1)): the first r workers take q + 1
// iterations, the others q (I = q W + r; all 32-bit, I < 2^31).
__device__ __forceinline__ uint32_t streamk_start(const StreamKParams &sk, uint32_t w)
{
    return w * sk.q + (w < sk.r ? w : sk.r);
}

// The worker whose range holds iteration i.
__device__ __forceinline__ uint32_t streamk_owner(const StreamKParams &sk, uint32_t i)
{
    const uint32_t big = sk.r * (sk.q + 1); // iterations of the first r workers
    return i < big ? i / (sk.q + 1) : sk.r + (i - big) / sk.q;
}

// Thread 0 of a finisher waits (bounded) for worker v's flag and clears it.  A
// wait that gives up sets the error word and leaves the flag as the late worker
// leaves it: the error word tells the caller to clear the workspace again.
__device__ __forceinline__ void wait_flag(const StreamKParams &sk, uint32_t v)
{
    uint32_t n = 0;
    while (__hip_atomic_load(&sk.flags[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(4);
        if (++n >= sk.spin_limit) {
            __hip_atomic_store(sk.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
    __hip_atomic_store(&sk.flags[v], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int T, int O, int BM, int BN, int WGM, int WGN, int AMODE, int BMODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
    __attribute__((amdgpu_waves_per_eu(2, 2))) gemm_streamk(GemmParams p, StreamKParams sk)
{
    typedef Tiled<T, O, BM, BN, WGM, WGN, AMODE, BMODE> G;
    typedef typename G::acc_t acc_t;
    __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE];

    const uint32_t tid = threadIdx.x;
    const uint32_t w = xcd_remap(sk.workers, blockIdx.x); // consecutive ranges share an XCD
    const uint32_t nk = sk.nk;
    const uint32_t s0 = streamk_start(sk, w), e0 = streamk_start(sk, w + 1);
    phase_begin(p.phases, w, e0 > s0 ? e0 - s0 : 0u);
    if (s0 >= e0) {
        phase_mark(p.phases, w, PH_LOOP);
        phase_mark(p.phases, w, PH_FIX);
        phase_end(p.phases, w);
        return; // more workers than iterations
    }

    const uint32_t t_lo = s0 / nk, t_hi = (e0 - 1) / nk;
    for (uint32_t t = t_hi + 1; t-- > t_lo;) {
        const uint32_t ts = t * nk;
        const int kb = (int)((s0 > ts ? s0 : ts) - ts);
        const int ke = (int)((e0 < ts + nk ? e0 : ts + nk) - ts);
        acc_t acc[G::MT][G::NT];
#pragma unroll
        for (int i = 0; i < G::MT; ++i)
#pragma unroll
            for (int j = 0; j < G::NT; ++j)
                acc[i][j] = acc_t{};
        const TileCoord tc = tile_coord(p, t);
        uint32_t tid_m = threadIdx.x;
        asm volatile("" : "+v"(tid_m));
        typename G::Staging st;
        G::mainloop(p, tc, kb, ke, smem, acc, tid_m, st);
        uint32_t tid_e = threadIdx.x; // the lane arithmetic of what follows, afresh
        asm volatile("" : "+v"(tid_e));
        const uint32_t lane = tid_e & 63u, wave = __builtin_amdgcn_readfirstlane(tid_e >> 6);
        phase_mark(p.phases, w, PH_LOOP);

        if ((uint32_t)ke < nk) {
            phase_mark(p.phases, w, PH_FIX);
            // not the finisher: the leading part of tile t, for a higher worker
            G::store_partial(sk.partials + (size_t)w * G::PARTIAL_BYTES, acc, lane, wave);
            // each wavefront's device-coherent stores have completed, then the flag
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(&sk.flags[w], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (kb > 0) { // the lower workers that hold K-tiles [0, kb) of this tile
                // Their partials are added in increasing worker order (the same bits on
                // every run), a whole slot per round trip -- two slots at once when the
                // registers allow it (up to 32 accumulator registers per slot).
                constexpr uint32_t STEP = G::MT * G::NT <= 8 ? 2u : 1u;
                for (uint32_t v = streamk_owner(sk, ts); v < w; v += STEP) {
                    const bool two = STEP == 2 && v + 1 < w;
                    if (tid == 0) {
                        wait_flag(sk, v);
                        if (two)
                            wait_flag(sk, v + 1);
                    }
                    __syncthreads(); // the device-coherent loads below are issued after the flags were seen
                    acc_t x[G::MT][G::NT];
                    G::load_partial(sk.partials + (size_t)v * G::PARTIAL_BYTES, x, lane, wave);
                    if constexpr (STEP == 2) {
                        acc_t y[G::MT][G::NT];
                        if (two)
                            G::load_partial(sk.partials + (size_t)(v + 1) * G::PARTIAL_BYTES, y, lane, wave);
                        G::add_into(acc, x);
                        if (two)
                            G::add_into(acc, y);
                    } else {
                        G::add_into(acc, x);
                    }
                }
            }
            __syncthreads(); // every wavefront is done with the stages before the parking
            phase_mark(p.phases, w, PH_FIX);
            G::epilogue(p, tc, acc, smem, lane, wave);
        }
        __syncthreads(); // the next tile's prologue overwrites the stages
    }
    phase_end(p.phases, w);
}

} // namespace dmu
