// Tile scheduling and ring bookkeeping, host+device so the CPU tests can
// evaluate exactly what the kernels run.
//
// Tile decomposition: output tile (m_idx, n_idx) covers
// D[m_idx*BM .. +BM, n_idx*BN .. +BN], reads A rows m_idx*BM.. and B rows
// n_idx*BN.. ("TIRx GEMM detailed technical notes", V3 "Spatial Tiling with
// Multiple CTAs": m_st = bx*BLK_M, n_st = by*BLK_N).
//
// Grouped order: the persistent scheduler of the same notes (V6 "Better L2
// Locality") visits tiles in groups of 8 along M so that neighbouring tiles
// share A row bands and B row bands in L2.  The notes give no formula; the
// reading used here walks a group of (up to) 8 tile rows column by column.
//
// XCD remap: a gfx950 device dispatches consecutive workgroups round-robin
// over its 8 XCDs, each with a private L2.  Workgroup w is given slot
// xcd_slot(w) so that the workgroups resident on one XCD take a contiguous
// run of the grouped order.  Both maps are bijections for any grid size, so
// the result never depends on them (only the L2 hit rate does).
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#define __host__
#define __device__
#define __forceinline__ inline
#endif

namespace g16 {

constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;

struct TileCoord {
    int64_t m_idx, n_idx;
};

// Grouped order with groups of `group_m` tile rows, in the integer type I:
// linear tile id t -> tile row *m_idx and tile column *n_idx.  Group g
// holds tile rows [g*group_m, g*group_m + gm), gm = group_m except for a
// shorter last group, walked column by column.  The four-wave ring runs it
// in 32-bit arithmetic with groups of 4 (kRing4GroupM in ring4.hpp), the
// other persistent and grouped rungs with kGroupM in 64-bit.
template <typename I>
__host__ __device__ __forceinline__ void grouped_tile_in(I t, I tiles_m, I tiles_n, I group_m, I* m_idx, I* n_idx)
{
    const I per_group = group_m * tiles_n;
    const I g = t / per_group;
    const I first_m = g * group_m;
    const I rem = tiles_m - first_m;
    const I gm = rem < group_m ? rem : group_m;
    const I r = t - g * per_group;
    *m_idx = first_m + r % gm;
    *n_idx = r / gm;
}

// Linear tile id t (grouped order, groups of kGroupM) -> tile coordinates.
__host__ __device__ __forceinline__ TileCoord grouped_tile(int64_t t, int64_t tiles_m, int64_t tiles_n)
{
    TileCoord c;
    grouped_tile_in<int64_t>(t, tiles_m, tiles_n, (int64_t)kGroupM, &c.m_idx, &c.n_idx);
    return c;
}

// First output row (or column) of tile `idx` along an extent of `extent`
// elements cut in tiles of `tile` (extent >= tile): the last tile is moved
// back to end at the extent, so every tile is whole and in range (it
// overlaps its neighbour, which computes the same values for the shared
// rows).  The four-wave ring's tiles; the other rungs mask their edges.
__host__ __device__ __forceinline__ int64_t clamped_origin(int64_t idx, int64_t tile, int64_t extent)
{
    const int64_t o = idx * tile;
    return o < extent - tile ? o : extent - tile;
}

// Workgroup id -> slot in [0, grid) such that the workgroups dispatched to
// one XCD (w mod 8 equal) own one contiguous range of slots.
__host__ __device__ __forceinline__ int64_t xcd_slot(int64_t w, int64_t grid)
{
    const int64_t x = w % kNumXcd;
    const int64_t j = w / kNumXcd;
    const int64_t q = grid / kNumXcd;
    const int64_t r = grid % kNumXcd;
    return x * q + (x < r ? x : r) + j;
}

// The i-th tile visited by workgroup w of a persistent grid of `grid`
// workgroups, as a linear grouped-order id; >= total when done.
__host__ __device__ __forceinline__ int64_t persistent_tile(int64_t w, int64_t i, int64_t grid)
{
    return xcd_slot(w, grid) + i * grid;
}

// Ring bookkeeping for a ring of `depth` stages fed with k-steps 0, 1, ...:
// step k lives in stage k % depth and is the (k / depth)-th use of that
// stage ("lap"; the pages' phase bit is lap & 1).  With one counter per ring
// that never resets, a wait always names the current lap, including across
// tile boundaries of the persistent kernels.
__host__ __device__ __forceinline__ int ring_stage(int64_t k, int depth) { return (int)(k % depth); }
__host__ __device__ __forceinline__ int64_t ring_lap(int64_t k, int depth) { return k / depth; }

// Refill rule of the software pipeline ("TIRx GEMM detailed technical
// notes", V5 "Main-Loop Schedule"): once step k has been consumed, its stage
// is refilled with step k + depth, if that step exists.  Returns -1 when
// nothing is left.  The kernels issue this refill at the barrier that opens
// step k + 1 (k = -1 there stands for the prologue, which fills steps
// 0 .. depth-2 before the loop, so step depth-1 is issued on entry).
__host__ __device__ __forceinline__ int64_t ring_refill_after(int64_t k, int depth, int64_t total)
{
    const int64_t p = k + depth;
    return p < total ? p : -1;
}

// Producer/consumer handoff of the wave-specialized ring (rung 5), the
// pages' two mbarrier rings ("GEMM III", Step 7 "Four barriers = two
// producer-consumer rings") as two monotonic counters per stage in LDS:
// every producer wave adds 1 to ready[s] once its loads of a step in stage
// s have landed, every consumer wave adds 1 to free[s] once it has read
// the step.  The counters never reset (across tiles either), so each wait
// names an absolute count and can never be satisfied by an earlier lap:
//   a consumer reads step k once ready[k % depth] >= ready_target(k);
//   a producer refills stage k % depth with step k once
//   free[k % depth] >= free_target(k) (all consumers are done with step
//   k - depth; 0 for the first lap, so the producers start with every
//   stage free and the consumers start blocked -- the pages' opposite
//   initial phases).
__host__ __device__ __forceinline__ uint32_t handoff_ready_target(int64_t k, int depth, int producers)
{
    return (uint32_t)producers * (uint32_t)(k / depth + 1);
}
__host__ __device__ __forceinline__ uint32_t handoff_free_target(int64_t k, int depth, int consumers)
{
    return (uint32_t)consumers * (uint32_t)(k / depth);
}
// Whether a counter has reached a target (signed distance: the counters
// may wrap around 2^32 in a very long persistent run).
__host__ __device__ __forceinline__ bool handoff_reached(uint32_t counter, uint32_t target)
{
    return (int32_t)(counter - target) >= 0;
}

}  // namespace g16
