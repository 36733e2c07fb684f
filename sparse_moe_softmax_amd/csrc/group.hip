// GPU-resident grouping of routed slots by expert: histogram, prefix-sum
// offsets, stable permutation and tile block map, with no host round trip.
// The pages keep the routing histograms and block maps on the GPU so that no
// CPU-GPU synchronisation is needed between routing and the expert GEMMs
// (Inside Lily page, section "Performance Gains and Workload Patterns").
//
// Three steps, all on the device:
//   1. per routing tile (kTopkTile tokens): expert histogram          (k_tile_hist, or fused into k_topk)
//   2. per expert: exclusive scan of its count over the tiles  (k_group_scan, one block per expert)
//   3. per tile: stable in-tile ranks from wavefront ballots,
//      positions = offsets[e] + tile base + rank               (k_group_scatter)
// Up to 64 routing tiles (T <= 1024 with 16-token tiles) steps 2 and 3 run
// as one launch (k_group_fused), each block forming its own column sums.
// Integer counting only, so every output is bitwise deterministic.  An id
// outside [0, E) (possible only for caller-supplied ids) is skipped: it is not
// counted, its slot gets no position (inv_perm -1), and the MOE_DEVERR_EXPERT_ID
// bit is set in the error word when one is given.
#include "internal.hpp"

namespace moe {

__device__ inline void flag_bad_id(uint32_t* err) {
  if (err)
    __hip_atomic_fetch_or(err, static_cast<uint32_t>(MOE_DEVERR_EXPERT_ID), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_tile_hist(const int32_t* __restrict__ ids, int T, int k, int E,
                                                   int32_t* __restrict__ tilehist, uint32_t* __restrict__ err) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kTopkTile * k;
  const int64_t f1 = min(static_cast<int64_t>(T) * k, f0 + static_cast<int64_t>(kTopkTile) * k);
  for (int64_t f = f0 + threadIdx.x; f < f1; f += 256) {
    const int e = ids[f];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E))
      atomicAdd(&hist[e], 1);
    else
      flag_bad_id(err);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) tilehist[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

hipError_t launch_tile_hist(const int32_t* ids, int T, int k, int E, int32_t* tilehist, uint32_t* err,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_tile_hist, dim3(static_cast<unsigned>(div_up(T, kTopkTile))), dim3(256), 0, s, ids, T, k, E,
                     tilehist, err);
  return hipGetLastError();
}

// Exclusive scan of one value per thread over a 256-thread block; returns the
// exclusive prefix and writes the block total to *total.
__device__ inline int block_excl_scan256(int v, int* sm, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sm[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += sm[w];
  const int tot = sm[0] + sm[1] + sm[2] + sm[3];
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

// Block e: exclusive prefix of tilehist[.][e] over the tiles -> tilebase, total -> counts[e].
__global__ __launch_bounds__(256) void k_group_scan(const int32_t* __restrict__ tilehist,
                                                    int32_t* __restrict__ tilebase, int ntile, int E,
                                                    int32_t* __restrict__ counts) {
  __shared__ int sm[4];
  const int e = blockIdx.x;
  int carry = 0;
  for (int base = 0; base < ntile; base += 256) {
    const int i = base + threadIdx.x;
    const int v = (i < ntile) ? tilehist[static_cast<int64_t>(i) * E + e] : 0;
    int tot;
    const int ex = block_excl_scan256(v, sm, &tot);
    if (i < ntile) tilebase[static_cast<int64_t>(i) * E + e] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// The rest of the grouping for routing tile blockIdx.x, given per expert e =
// threadIdx.x its slot count c, the exclusive prefix off of the counts, their
// total, and base[e] = offsets[e] + the slots of expert e in earlier tiles,
// already in LDS.  With write_map (or tile_rows), block 0 writes offsets, the
// block map and n_tiles (and the rows of every tile).  Wave 0 then walks the
// tile's flat slots in order, 64 at a time: lanes with equal expert id find
// each other through 8 ballots (one per id bit), the rank of a lane is the
// number of matching lower lanes, and the group's count advances base[e].
__device__ inline void group_place(int c, int off, int total, int* base, int* sm, const int32_t* __restrict__ ids,
                                   int T, int k, int E, int block_m, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                   int32_t* __restrict__ block_map, int max_tiles, int32_t* __restrict__ n_tiles,
                                   int write_map, int32_t* __restrict__ tile_rows, uint32_t* __restrict__ err) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && (write_map || tile_rows)) {
    const int nt = (c + block_m - 1) / block_m;
    int nt_total;
    const int toff = block_excl_scan256(nt, sm, &nt_total);
    // rows of every tile, so that a GEMM tile learns its height in the same
    // round trip as its block-map entry
    if (tile_rows && tid < E)
      for (int m = 0; m < nt; ++m) tile_rows[toff + m] = min(block_m, c - m * block_m);
    if (write_map) {
      if (tid < E) {
        offsets[tid] = off;
        for (int m = 0; m < nt; ++m) {
          block_map[2 * (toff + m)] = tid;
          block_map[2 * (toff + m) + 1] = off + m * block_m;
        }
      }
      if (tid == 0) {
        offsets[E] = total;
        *n_tiles = nt_total;
      }
      for (int i = nt_total + tid; i < max_tiles; i += 256) {
        block_map[2 * i] = -1;
        block_map[2 * i + 1] = -1;
      }
    }
  }
  __syncthreads();

  if (tid < 64) {
    const int lane = tid;
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kTopkTile * k;
    const int64_t f1 = min(static_cast<int64_t>(T) * k, f0 + static_cast<int64_t>(kTopkTile) * k);
    for (int64_t fb = f0; fb < f1; fb += 64) {
      const int64_t f = fb + lane;
      const bool in_tile = f < f1;
      const int id = in_tile ? ids[f] : 0;
      const bool valid = in_tile && static_cast<unsigned>(id) < static_cast<unsigned>(E);
      if (in_tile && !valid) {
        inv_perm[f] = -1;
        flag_bad_id(err);
      }
      const int e = valid ? id : 0;
      uint64_t match = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t bal = __ballot((e >> b) & 1);
        match &= ((e >> b) & 1) ? bal : ~bal;
      }
      const int rank = __popcll(match & lt);
      const int pos = base[e] + rank;  // every lane reads before any lane updates
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        perm[pos] = static_cast<int32_t>(f);
        inv_perm[f] = pos;
        if (rank == 0) base[e] = pos + __popcll(match);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Block b = routing tile b.  All threads: offsets = exclusive scan of counts,
// running base[e] = offsets[e] + tilebase[b][e]; then group_place.
__global__ __launch_bounds__(256) void k_group_scatter(const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ tilebase, int T, int k, int E,
                                                       int block_m, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                                       int32_t* __restrict__ block_map, int max_tiles,
                                                       int32_t* __restrict__ n_tiles, int write_map,
                                                       int32_t* __restrict__ tile_rows, uint32_t* __restrict__ err) {
  __shared__ int base[256];
  __shared__ int sm[4];
  const int tid = threadIdx.x;
  const int c = (tid < E) ? counts[tid] : 0;
  int total;
  const int off = block_excl_scan256(c, sm, &total);
  if (tid < E) base[tid] = off + tilebase[static_cast<int64_t>(blockIdx.x) * E + tid];
  group_place(c, off, total, base, sm, ids, T, k, E, block_m, offsets, perm, inv_perm, block_map, max_tiles, n_tiles,
              write_map, tile_rows, err);
}

// Steps 2 and 3 in one launch, for up to kFusedTiles routing tiles: block b
// sums every tile's histogram column of its expert (thread e) itself, the
// tiles before b separately, so the per-expert scan needs no launch of its
// own (each block reads the whole ntile x E histogram, at most 64 KB, from
// L2).  Block 0 also writes counts.  At 256 tiles (T = 4096) those reads cost
// more than the launch they save (grouping 11.7 -> 17.9 us); at 4 and 32
// tiles the grouping goes from 11.2 to 8.2 us.
constexpr int kFusedTiles = 64;
__global__ __launch_bounds__(256) void k_group_fused(const int32_t* __restrict__ ids,
                                                     const int32_t* __restrict__ tilehist, int ntile, int T, int k,
                                                     int E, int block_m, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv_perm, int32_t* __restrict__ block_map,
                                                     int max_tiles, int32_t* __restrict__ n_tiles,
                                                     int32_t* __restrict__ tile_rows, uint32_t* __restrict__ err) {
  __shared__ int base[256];
  __shared__ int sm[4];
  const int tid = threadIdx.x, b = blockIdx.x;
  int pre = 0, c = 0;
  if (tid < E) {
    const int32_t* col = tilehist + tid;
#pragma unroll 8
    for (int i = 0; i < b; ++i) pre += col[static_cast<int64_t>(i) * E];
    c = pre;
#pragma unroll 8
    for (int i = b; i < ntile; ++i) c += col[static_cast<int64_t>(i) * E];
  }
  int total;
  const int off = block_excl_scan256(c, sm, &total);
  if (tid < E) {
    base[tid] = off + pre;
    if (b == 0) counts[tid] = c;
  }
  group_place(c, off, total, base, sm, ids, T, k, E, block_m, offsets, perm, inv_perm, block_map, max_tiles, n_tiles,
              1, tile_rows, err);
}

hipError_t launch_group_counts(const int32_t* tilehist, int32_t* tilebase, int T, int E, int32_t* counts,
                               hipStream_t s) {
  const int ntile = static_cast<int>(div_up(T, kTopkTile));
  hipLaunchKernelGGL(k_group_scan, dim3(E), dim3(256), 0, s, tilehist, tilebase, ntile, E, counts);
  return hipGetLastError();
}

hipError_t launch_group_scatter(const int32_t* ids, const int32_t* counts, const int32_t* tilebase, int T, int k,
                                int E, int block_m, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* block_map, int max_tiles, int32_t* n_tiles, bool write_map,
                                int32_t* tile_rows, uint32_t* err, hipStream_t s) {
  const int ntile = static_cast<int>(div_up(T, kTopkTile));
  hipLaunchKernelGGL(k_group_scatter, dim3(ntile), dim3(256), 0, s, ids, counts, tilebase, T, k, E, block_m, offsets,
                     perm, inv_perm, block_map, max_tiles, n_tiles, write_map ? 1 : 0, tile_rows, err);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* ids, const int32_t* tilehist, int32_t* tilebase, int T, int k, int E,
                        int block_m, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* block_map, int max_tiles, int32_t* n_tiles, int32_t* tile_rows, uint32_t* err,
                        hipStream_t s) {
  const int ntile = static_cast<int>(div_up(T, kTopkTile));
  if (ntile <= kFusedTiles) {
    hipLaunchKernelGGL(k_group_fused, dim3(ntile), dim3(256), 0, s, ids, tilehist, ntile, T, k, E, block_m, counts,
                       offsets, perm, inv_perm, block_map, max_tiles, n_tiles, tile_rows, err);
    return hipGetLastError();
  }
  const hipError_t e = launch_group_counts(tilehist, tilebase, T, E, counts, s);
  if (e != hipSuccess) return e;
  return launch_group_scatter(ids, counts, tilebase, T, k, E, block_m, offsets, perm, inv_perm, block_map, max_tiles,
                              n_tiles, true, tile_rows, err, s);
}

}  // namespace moe
