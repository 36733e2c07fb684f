// Wave-level top-k with a compile-time k, shared by the routing kernel of the
// grouped path and the fused decode layer.  Each token keeps its k best-scored
// experts (Lily page, section "The architecture that forces the issue: MoE
// plus Gated DeltaNet"); the order is larger logit first, lower expert index
// among equal logits, -0 and +0 equal.
#pragma once
#include "internal.hpp"

namespace moe {

// Largest of a 32-bit value over the whole wave, in lane 63: maximum within
// each 16-lane row (DPP), then row 0 broadcast into row 1 and row 2 into row 3
// (row_bcast:15), then row 1 into rows 2 and 3 (row_bcast:31).
__device__ inline uint32_t wave_max_u32_lane63(uint32_t v) {
  v = row_max16_u32(v);
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x142, 0xA,
                                                                0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x143, 0xC,
                                                                0xF, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Top-K for a compile-time K, the same selection as topk_wave64_regs (larger
// key first, lowest expert index among equal keys): K straight-line rounds,
// each one wave maximum and four ballots.  Lane r < K ends with slot r's
// expert and logit.
template <int K>
__device__ inline void topk_wave64_fixed(const float (&v)[4], int E, int& my_e, float& my_v) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = lane + 64 * i < E ? topk_key32(v[i]) : 0u;
  my_e = 0;
  my_v = 0.f;
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const uint32_t best = wave_max_u32_lane63(max(max(key[0], key[1]), max(key[2], key[3])));
    const uint64_t b0 = __ballot(key[0] == best), b1 = __ballot(key[1] == best);
    const uint64_t b2 = __ballot(key[2] == best), b3 = __ballot(key[3] == best);
    // lowest matching expert index: the first non-empty ballot, its lowest lane
    const uint32_t c0 = b0 ? static_cast<uint32_t>(__builtin_ctzll(b0)) : ~0u;
    const uint32_t c1 = b1 ? 64u + static_cast<uint32_t>(__builtin_ctzll(b1)) : ~0u;
    const uint32_t c2 = b2 ? 128u + static_cast<uint32_t>(__builtin_ctzll(b2)) : ~0u;
    const uint32_t c3 = b3 ? 192u + static_cast<uint32_t>(__builtin_ctzll(b3)) : ~0u;
    const int e = static_cast<int>(min(min(c0, c1), min(c2, c3)));
    const bool here = lane == (e & 63);
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = (here && (e >> 6) == i) ? 0u : key[i];
    if (lane == r) {
      my_e = e;
      my_v = topk_key32_value(best);
    }
  }
}

}  // namespace moe
