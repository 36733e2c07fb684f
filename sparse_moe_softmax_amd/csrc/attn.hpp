// attn.hpp -- host-side plan and launch of the grouped-query decode attention (attn.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

// The positions of a sequence are cut into n_splits ranges of rows_per_split;
// a workgroup takes heads_per_wg query heads.
struct GqaPlan {
  int heads_per_wg;
  int rows_per_split;
  int n_splits;
};
GqaPlan gqa_plan(int B, int Hq, int Hkv, int S, bool packed);
size_t gqa_workspace_bytes(int B, int Hq, int Hkv, int S, int D);
hipError_t launch_gqa_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* lens, int B,
                             int Hq, int Hkv, int D, int S, float scale, bool packed, uint16_t* out, void* workspace,
                             hipStream_t s);

}  // namespace moe
