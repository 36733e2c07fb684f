// Drives the C ABI's host code (argument checks, workspace carving, the host
// block map, the error and residency queries) in a build whose host code has
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py).
// Without a GPU every launch path ends in MOE_ERR_HIP; the device pointers
// passed here are never dereferenced on the host.  On a machine with a GPU
// the launch paths are skipped (the fake device pointers would fault).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/moe.h"

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(1);                                                       \
    }                                                                     \
  } while (0)

int main() {
  int n_dev = 0;
  const bool gpu = hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0;
  const moe_dims d = {2048, 512, 256, 8, 64, 512};
  void* F = reinterpret_cast<void*>(uintptr_t{4096});   // a device pointer never dereferenced here
  for (int32_t s : {0, -1, -2, -3, -4, -5, 7, INT32_MIN, INT32_MAX}) CHECK(moe_status_str(s) != nullptr);
  CHECK(moe_block_m() == 128);
  CHECK(moe_max_tiles(4096, 8, 256, 128) == 512);
  CHECK(moe_max_tiles(-1, 8, 256, 128) == 0);
  // sizes
  for (int T : {1, 4, 5, 64, 4096, 65536}) {
    CHECK(moe_workspace_bytes(&d, T) > 0);
    CHECK(moe_group_workspace_bytes(&d, T) >= 256);
    CHECK(moe_host_routing_bytes(&d, T) > 0);
  }
  CHECK(moe_workspace_bytes(&d, 0) == 0 && moe_workspace_bytes(nullptr, 4) == 0);
  for (int m = 0; m < 4; ++m) CHECK(moe_packed_q4_bytes(&d, m, 3) > 0);
  CHECK(moe_packed_q4_bytes(&d, 4, 1) == 0);
  CHECK(moe_gqa_decode_workspace_bytes(1, 16, 2, 256, 32768) > 0);
  CHECK(moe_gqa_decode_workspace_bytes(1, 16, 2, 96, 100) == 0);
  // host block map against a direct loop, and its checks
  const int E = 37, bm = 7;
  std::vector<int32_t> counts(E);
  for (int e = 0; e < E; ++e) counts[e] = (e * 13) % 17;
  const int mt = moe_max_tiles(64, 8, E, bm);
  std::vector<int32_t> off(E + 1), bmap(2 * mt);
  int32_t nt = -1;
  CHECK(moe_host_block_map(counts.data(), E, bm, mt, off.data(), bmap.data(), &nt) == MOE_OK);
  int tiles = 0, o = 0;
  for (int e = 0; e < E; ++e) {
    CHECK(off[e] == o);
    for (int r = 0; r < counts[e]; r += bm, ++tiles) CHECK(bmap[2 * tiles] == e && bmap[2 * tiles + 1] == o + r);
    o += counts[e];
  }
  CHECK(nt == tiles && off[E] == o);
  for (int i = tiles; i < mt; ++i) CHECK(bmap[2 * i] == -1 && bmap[2 * i + 1] == -1);
  CHECK(moe_host_block_map(counts.data(), E, bm, tiles - 1, off.data(), bmap.data(), &nt) == MOE_ERR_INVALID_ARG);
  counts[3] = -1;
  CHECK(moe_host_block_map(counts.data(), E, bm, mt, off.data(), bmap.data(), &nt) == MOE_ERR_INVALID_ARG);
  CHECK(moe_host_block_map(nullptr, E, bm, mt, off.data(), bmap.data(), &nt) == MOE_ERR_INVALID_ARG);
  // argument checks of every entry point
  const moe_dims bad_g = {2048, 512, 256, 8, 32, 512}, bad_k = {2048, 512, 256, 17, 64, 512};
  int32_t* I32 = static_cast<int32_t*>(F);
  float* F32 = static_cast<float*>(F);
  uint16_t* U16 = static_cast<uint16_t*>(F);
  CHECK(moe_route(&bad_g, F32, nullptr, 4, I32, F32, nullptr, nullptr) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_route(&bad_k, F32, nullptr, 4, I32, F32, nullptr, nullptr) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_route(&d, F32, nullptr, 0, I32, F32, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_route(&d, nullptr, nullptr, 4, I32, F32, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_group(&d, I32, 100, 0, I32, I32, I32, I32, I32, 1000, I32, F, 1 << 20, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_group(&d, I32, 100, 64, I32, I32, I32, I32, I32, 2, I32, F, 1 << 20, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_group(&d, I32, 100, 64, I32, I32, I32, I32, I32, 1000, I32, F, 16, nullptr) == MOE_ERR_WORKSPACE);
  const moe_q4 q = {static_cast<const uint8_t*>(F), U16, U16, static_cast<const uint8_t*>(F)};
  const moe_q4 unpacked = {static_cast<const uint8_t*>(F), U16, U16, nullptr};
  CHECK(moe_grouped_gemm_q4(&d, &q, MOE_EPI_SWIGLU_BF16, U16, 2, I32, I32, I32, I32, 10, nullptr, 100, 64, F,
                            nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_grouped_gemm_q4(&d, &unpacked, MOE_EPI_SWIGLU_BF16, U16, 1, I32, I32, I32, I32, 10, nullptr, 100, 64, F,
                            nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_grouped_gemm_q4(&d, &q, MOE_EPI_WEIGHTED_SCATTER_F32, U16, 0, I32, I32, I32, I32, 10, nullptr, 100, 64,
                            F, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_grouped_gemm_q4(&d, &q, 7, U16, 0, I32, I32, I32, I32, 10, F32, 100, 64, F, nullptr) ==
        MOE_ERR_INVALID_ARG);
  const moe_layer L = {q, q, q, q, F32, nullptr, F32, U16};
  const size_t need = moe_workspace_bytes(&d, 4096);
  CHECK(moe_forward(&d, &L, U16, 4096, U16, nullptr, nullptr, nullptr, F, need - 1, nullptr) == MOE_ERR_WORKSPACE);
  CHECK(moe_forward(&d, nullptr, U16, 4096, U16, nullptr, nullptr, nullptr, F, need, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_forward_stages(&d, &L, U16, 64, U16, nullptr, nullptr, nullptr, F, need, 4, 2, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_forward_noalloc(&d, &L, U16, 1024, U16, nullptr, nullptr, nullptr, nullptr) == MOE_ERR_WORKSPACE);
  int32_t flags = 0, n = 0, r = 0;
  CHECK(moe_workspace_errors(nullptr, 1024, 0, &flags, nullptr) == MOE_ERR_WORKSPACE);
  CHECK(moe_workspace_errors(F, 1024, 0, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fused_residency(&d, 5, &n, &r) == MOE_ERR_UNSUPPORTED);
  std::vector<uint8_t> hb(moe_host_routing_bytes(&d, 512));
  CHECK(moe_forward_host_routing(&d, &L, U16, 3, U16, nullptr, nullptr, F, need, hb.data(), hb.size(), nullptr) ==
        MOE_ERR_UNSUPPORTED);
  CHECK(moe_gqa_decode_attention(U16, U16, U16, I32, 2, 16, 3, 128, 1000, 0.1f, 1, U16, F, 1 << 20, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_last_error_message() != nullptr);
  if (!gpu) {
    // past validation every path meets the missing device as a HIP error
    CHECK(moe_fused_residency(&d, 1, &n, &r) == MOE_ERR_HIP);
    CHECK(moe_forward(&d, &L, U16, 1, U16, nullptr, nullptr, nullptr, F, need, nullptr) == MOE_ERR_HIP);
    CHECK(moe_forward(&d, &L, U16, 4096, U16, nullptr, nullptr, nullptr, F, need, nullptr) == MOE_ERR_HIP);
    CHECK(moe_forward_noalloc(&d, &L, U16, 64, U16, nullptr, nullptr, nullptr, nullptr) == MOE_ERR_HIP);
    CHECK(moe_group(&d, I32, 100, 64, I32, I32, I32, I32, I32, 1000, I32, F, 1 << 20, nullptr) == MOE_ERR_HIP);
    CHECK(moe_workspace_errors(F, 1024, 1, &flags, nullptr) == MOE_ERR_HIP);
    CHECK(moe_last_hip_error() != 0);
  }
  std::printf("abi driver: ok (%s)\n", gpu ? "device present: launch paths skipped" : "no device");
  return 0;
}
