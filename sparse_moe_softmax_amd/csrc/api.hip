// C ABI of libmoe: argument validation, workspace carving and the launch
// sequence of every entry point.  Nothing here synchronises the host with the
// device and nothing allocates device memory.
#include <algorithm>
#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.hpp"
#include "attn.hpp"

using namespace moe;

namespace {

thread_local char g_msg[256] = "";
thread_local int32_t g_hip_err = 0;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

moe_status hip_check(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  g_hip_err = static_cast<int32_t>(e);
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

moe_status check_dims(const moe_dims* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
  if (d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->group_size <= 0 ||
      d->shared_inter <= 0)
    return fail(MOE_ERR_INVALID_ARG, "dims must be positive");
  if (d->group_size != 64) return fail(MOE_ERR_UNSUPPORTED, "group_size must be 64");
  if (d->hidden % 64) return fail(MOE_ERR_UNSUPPORTED, "hidden must be a multiple of 64");
  if (d->inter % 64 || d->shared_inter % 64)
    return fail(MOE_ERR_UNSUPPORTED, "inter and shared_inter must be multiples of 64");
  if (d->n_experts % 16 || d->n_experts > 256) return fail(MOE_ERR_UNSUPPORTED, "n_experts must be 16..256, x16");
  if (d->top_k > 16 || d->top_k > d->n_experts) return fail(MOE_ERR_UNSUPPORTED, "top_k must be <= 16 and <= n_experts");
  return MOE_OK;
}

moe_status check_T(int32_t T) {
  if (T < 1 || T > 65536) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [1, 65536]", T);
  return MOE_OK;
}

moe_status check_q4(const moe_q4* q, const char* name) {
  if (!q || !q->codes || !q->scales || !q->biases) return fail(MOE_ERR_INVALID_ARG, "%s: NULL weight pointer", name);
  return MOE_OK;
}

moe_status check_packed(const moe_q4* q, const char* name) {
  if (!q || !q->packed) return fail(MOE_ERR_INVALID_ARG, "%s: packed weights are NULL (run moe_prepack_q4)", name);
  return MOE_OK;
}

// The grouped GEMMs address activation rows with 32-bit byte offsets.
moe_status check_gemm_extent(const moe_dims& d, int32_t T) {
  const int64_t w = std::max(d.inter, d.shared_inter);
  if (static_cast<int64_t>(T) * d.hidden * 2 >= (int64_t{1} << 32) ||
      static_cast<int64_t>(T) * d.top_k * w * 2 >= (int64_t{1} << 32))
    return fail(MOE_ERR_UNSUPPORTED, "T=%d: activations of 4 GiB or more", T);
  return MOE_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Every workspace starts with this header; its first word is the device error word.
constexpr size_t kWsHeader = 256;

// Workspace regions of moe_forward.
struct Ws {
  size_t sync, logits, s, rparts, sparts, ids, wts, gate, tilehist, tilebase, counts, offsets, perm, inv, bmap, trows,
      ntiles, h, hsh, slots, sexp;
  int splits;
  size_t total;
};

Ws layout(const moe_dims& d, int32_t T) {
  const size_t E = d.n_experts, k = d.top_k, H = d.hidden, I = d.inter, Is = d.shared_inter;
  const size_t F = static_cast<size_t>(T) * k;
  const size_t ntile = static_cast<size_t>(div_up(T, kTopkTile));
  const size_t mt = static_cast<size_t>(moe_max_tiles(T, d.top_k, d.n_experts, kBM));
  Ws w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  take(kWsHeader);                       // error word
  w.sync = take(decode_sync_bytes(d));   // fused-path hand-over words, never written by the grouped path
  w.logits = take(T * E * 4);
  w.s = take(T * 4);
  w.splits = T > 1 ? router_splits(T, d.hidden, d.n_experts) : 1;
  w.rparts = take(w.splits > 1 ? w.splits * T * E * 4 : 0);
  w.sparts = take(w.splits > 1 ? w.splits * T * 4 : 0);
  w.ids = take(F * 4);
  w.wts = take(F * 4);
  w.gate = take(T * 4);
  w.tilehist = take(ntile * E * 4);
  w.tilebase = take(ntile * E * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.perm = take(F * 4);
  w.inv = take(F * 4);
  w.bmap = take(mt * 2 * 4);
  w.trows = take(mt * 4);
  w.ntiles = take(4);
  w.h = take(F * I * 2);
  w.hsh = take(static_cast<size_t>(T) * Is * 2);
  w.slots = take(static_cast<size_t>(T) * (k + 1) * H * 2);
  w.sexp = take(static_cast<size_t>(T) * (k + 1) * (H / 64));
  w.total = o;
  return w;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Residency of the fused layer's kernel on the current device, queried once
// per (device, dims, T) and kept.
std::mutex g_res_mu;
std::map<std::tuple<int, int, int, int, int, int, int>, std::pair<int, int>> g_res;

hipError_t fused_residency(const moe_dims& d, int T, int* needed, int* resident) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(dev, d.hidden, d.inter, d.shared_inter, d.n_experts, d.top_k, T);
  {
    std::lock_guard<std::mutex> lk(g_res_mu);
    auto it = g_res.find(key);
    if (it != g_res.end()) {
      *needed = it->second.first;
      *resident = it->second.second;
      return hipSuccess;
    }
  }
  e = decode_residency(d, T, needed, resident);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_res_mu);
  g_res[key] = {*needed, *resident};
  return hipSuccess;
}

__global__ void k_clear_word(uint32_t* w) { *w = 0u; }

}  // namespace

extern "C" {

int32_t moe_block_m(void) { return kBM; }

int32_t moe_max_tiles(int32_t T, int32_t top_k, int32_t n_experts, int32_t block_m) {
  if (T < 0 || top_k < 1 || n_experts < 1 || block_m < 1) return 0;
  return static_cast<int32_t>(div_up(static_cast<int64_t>(T) * top_k, block_m) + n_experts);
}

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error_message(void) { return g_msg; }
int32_t moe_last_hip_error(void) { return g_hip_err; }

moe_status moe_prepack_router(const moe_dims* d, const float* router_w, uint16_t* router_w3, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if (!router_w || !router_w3) return fail(MOE_ERR_INVALID_ARG, "NULL router weights");
  return hip_check(launch_prepack_router(router_w, router_w3, d->n_experts, d->hidden,
                                         static_cast<hipStream_t>(stream)),
                   "moe_prepack_router");
}

moe_status moe_router_logits(const moe_dims* d, const moe_layer* L, const uint16_t* x, int32_t T, float* logits,
                             float* shared_logit, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if (!L || !x || !logits) return fail(MOE_ERR_INVALID_ARG, "NULL layer, x or logits");
  if (shared_logit && !L->shared_gate_w) return fail(MOE_ERR_INVALID_ARG, "shared_logit needs shared_gate_w");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 1) {
    if (!L->router_w) return fail(MOE_ERR_INVALID_ARG, "router_w is NULL");
    return hip_check(launch_router_gemv(x, L->router_w, L->router_bias, L->shared_gate_w, 1, d->hidden,
                                        d->n_experts, logits, shared_logit, s),
                     "router gemv");
  }
  if (!L->router_w3) return fail(MOE_ERR_INVALID_ARG, "router_w3 is NULL (run moe_prepack_router)");
  return hip_check(launch_router_gemm(x, L->router_w3, L->router_bias, shared_logit ? L->shared_gate_w : nullptr, T,
                                      d->hidden, d->n_experts, 1, logits, shared_logit, s),
                   "router gemm");
}

moe_status moe_route(const moe_dims* d, const float* logits, const float* shared_logit, int32_t T, int32_t* ids,
                     float* weights, float* gate, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if (!logits || !ids || !weights) return fail(MOE_ERR_INVALID_ARG, "NULL logits, ids or weights");
  if ((gate != nullptr) != (shared_logit != nullptr))
    return fail(MOE_ERR_INVALID_ARG, "shared_logit and gate must both be given or both be NULL");
  return hip_check(launch_topk(logits, shared_logit, 1, nullptr, T, d->n_experts, d->top_k, nullptr, nullptr, ids,
                               weights, gate, nullptr, static_cast<hipStream_t>(stream)),
                   "top-k");
}

size_t moe_packed_q4_bytes(const moe_dims* d, int32_t matrix, int32_t n_exp) {
  if (check_dims(d) || matrix < MOE_MAT_GATE_UP || matrix > MOE_MAT_SH_DOWN || n_exp < 1) return 0;
  return static_cast<size_t>(pack_geom(*d, matrix).expert_bytes) * static_cast<size_t>(n_exp);
}

moe_status moe_prepack_q4(const moe_dims* d, int32_t matrix, const moe_q4* w, int32_t n_exp, uint8_t* packed,
                          size_t packed_bytes, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if (matrix < MOE_MAT_GATE_UP || matrix > MOE_MAT_SH_DOWN) return fail(MOE_ERR_INVALID_ARG, "unknown matrix %d", matrix);
  if (n_exp < 1) return fail(MOE_ERR_INVALID_ARG, "n_exp must be positive");
  if ((st = check_q4(w, "w"))) return st;
  if (!packed) return fail(MOE_ERR_INVALID_ARG, "packed is NULL");
  const size_t need = moe_packed_q4_bytes(d, matrix, n_exp);
  if (packed_bytes < need) return fail(MOE_ERR_INVALID_ARG, "packed_bytes %zu < %zu", packed_bytes, need);
  return hip_check(launch_prepack_q4(*d, matrix, *w, n_exp, packed, static_cast<hipStream_t>(stream)),
                   "moe_prepack_q4");
}

size_t moe_group_workspace_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) || check_T(T)) return 0;
  const size_t ntile = static_cast<size_t>(div_up(T, kTopkTile));
  return kWsHeader + 2 * align256(ntile * d->n_experts * 4);
}

moe_status moe_group(const moe_dims* d, const int32_t* ids, int32_t T, int32_t block_m, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* block_map, int32_t max_tiles,
                     int32_t* n_tiles, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if (!ids || !counts || !offsets || !perm || !inv_perm || !block_map || !n_tiles)
    return fail(MOE_ERR_INVALID_ARG, "NULL output pointer");
  if (block_m < 1 || block_m > 4096) return fail(MOE_ERR_INVALID_ARG, "block_m=%d outside [1, 4096]", block_m);
  if (max_tiles < moe_max_tiles(T, d->top_k, d->n_experts, block_m))
    return fail(MOE_ERR_INVALID_ARG, "max_tiles=%d < %d", max_tiles, moe_max_tiles(T, d->top_k, d->n_experts, block_m));
  const size_t need = moe_group_workspace_bytes(d, T);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t ntile = static_cast<size_t>(div_up(T, kTopkTile));
  uint32_t* err = at<uint32_t>(workspace, 0);
  int32_t* tilehist = at<int32_t>(workspace, kWsHeader);
  int32_t* tilebase = at<int32_t>(workspace, kWsHeader + align256(ntile * d->n_experts * 4));
  if ((st = hip_check(launch_tile_hist(ids, T, d->top_k, d->n_experts, tilehist, err, s), "tile histogram")))
    return st;
  return hip_check(launch_group(ids, tilehist, tilebase, T, d->top_k, d->n_experts, block_m, counts, offsets, perm,
                                inv_perm, block_map, max_tiles, n_tiles, nullptr, err, s),
                   "grouping");
}

moe_status moe_grouped_gemm_q4(const moe_dims* d, const moe_q4* w, int32_t epi, const uint16_t* a,
                               int32_t a_rows_are_tokens, const int32_t* perm, const int32_t* offsets,
                               const int32_t* block_map, const int32_t* n_tiles, int32_t max_tiles,
                               const float* row_weight, int32_t T, int32_t block_m, void* out, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if ((st = check_packed(w, "w"))) return st;
  if ((st = check_gemm_extent(*d, T))) return st;
  if (!a || !perm || !offsets || !block_map || !n_tiles || !out) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (block_m < 1 || block_m > kBM) return fail(MOE_ERR_INVALID_ARG, "block_m=%d outside [1, %d]", block_m, kBM);
  if (max_tiles < 1) return fail(MOE_ERR_INVALID_ARG, "max_tiles must be positive");
  if (a_rows_are_tokens != 0 && a_rows_are_tokens != 1)
    return fail(MOE_ERR_INVALID_ARG, "a_rows_are_tokens must be 0 or 1");
  const bool gather = a_rows_are_tokens == 1;
  {
    // rows of `a` are addressed with 32-bit byte offsets
    const int64_t rows = gather ? T : static_cast<int64_t>(T) * d->top_k;
    const int64_t K = epi == MOE_EPI_SWIGLU_BF16 ? d->hidden : d->inter;
    if (rows * K * 2 >= (int64_t{1} << 32)) return fail(MOE_ERR_UNSUPPORTED, "a: 4 GiB or more");
  }
  GemmTiles tl{perm, offsets, block_map, n_tiles, max_tiles, block_m, 0, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (epi == MOE_EPI_SWIGLU_BF16)
    return hip_check(launch_gemm_swiglu(*d, *w, nullptr, a, gather, tl, T, static_cast<uint16_t*>(out), nullptr, s),
                     "grouped gemm (swiglu)");
  if (epi == MOE_EPI_WEIGHTED_SCATTER_F32) {
    if (!row_weight) return fail(MOE_ERR_INVALID_ARG, "row_weight is NULL");
    return hip_check(launch_gemm_scatter(*d, *w, nullptr, a, gather, nullptr, tl, row_weight, nullptr, T,
                                         static_cast<float*>(out), s),
                     "grouped gemm (scatter)");
  }
  return fail(MOE_ERR_INVALID_ARG, "unknown epilogue %d", epi);
}

size_t moe_workspace_bytes(const moe_dims* d, int32_t T_max) {
  if (check_dims(d) || check_T(T_max)) return 0;
  return layout(*d, T_max).total;
}

moe_status moe_forward_stages(const moe_dims* d, const moe_layer* L, const uint16_t* x, int32_t T, uint16_t* y,
                              float* logits_out, int32_t* ids_out, float* w_out, void* workspace,
                              size_t workspace_bytes, int32_t first, int32_t last, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if (!L || !x || !y) return fail(MOE_ERR_INVALID_ARG, "NULL layer, x or y");
  if (first < MOE_STAGE_ROUTER || last > MOE_STAGE_COMBINE || first > last)
    return fail(MOE_ERR_INVALID_ARG, "stage range [%d, %d] invalid", first, last);
  // up to kDecMaxT tokens run as one fused launch on the canonical weights; the
  // grouped GEMMs read the packed ones
  const bool fused = T <= kDecMaxT && decode_supported(*d, T);
  auto chk = fused ? check_q4 : check_packed;
  if ((st = chk(&L->gate_up, "gate_up")) || (st = chk(&L->down, "down")) || (st = chk(&L->sh_gate_up, "sh_gate_up")) ||
      (st = chk(&L->sh_down, "sh_down")))
    return st;
  if (!L->shared_gate_w) return fail(MOE_ERR_INVALID_ARG, "shared_gate_w is NULL");
  const Ws w = layout(*d, T);
  if (!workspace || workspace_bytes < w.total)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, w.total);
  if (fused && !L->router_w) return fail(MOE_ERR_INVALID_ARG, "router_w is NULL");
  if (T == 1 && !fused)
    return fail(MOE_ERR_UNSUPPORTED, "T == 1 needs hidden <= 4096, inter and shared_inter <= 1024");
  if (!fused && !L->router_w3) return fail(MOE_ERR_INVALID_ARG, "router_w3 is NULL (run moe_prepack_router)");
  if (!fused && (st = check_gemm_extent(*d, T))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = logits_out ? logits_out : at<float>(workspace, w.logits);
  int32_t* ids = ids_out ? ids_out : at<int32_t>(workspace, w.ids);
  float* wts = w_out ? w_out : at<float>(workspace, w.wts);
  float* s_logit = at<float>(workspace, w.s);
  float* gate = at<float>(workspace, w.gate);
  auto run = [&](int stage) { return first <= stage && stage <= last; };

  uint32_t* err = at<uint32_t>(workspace, 0);
  if (fused) {
    // one launch for the whole layer, run as the ROUTER stage; its workgroups
    // wait for each other, so all of them must be resident at once
    int needed = 0, resident = 0;
    if ((st = hip_check(fused_residency(*d, T, &needed, &resident), "device query"))) return st;
    if (resident < needed)
      return fail(MOE_ERR_UNSUPPORTED, "the fused layer needs %d co-resident workgroups; the device holds %d", needed,
                  resident);
    DecodePtrs p{logits, s_logit, ids, wts, gate, at<void>(workspace, w.sync), err};
    if (run(MOE_STAGE_ROUTER)) return hip_check(launch_decode_layer(*d, *L, x, T, y, p, s), "fused layer");
    return MOE_OK;
  }
  uint16_t* slots = at<uint16_t>(workspace, w.slots);
  uint8_t* sexp = at<uint8_t>(workspace, w.sexp);
  int32_t* tilehist = at<int32_t>(workspace, w.tilehist);
  int32_t* counts = at<int32_t>(workspace, w.counts);
  int32_t* offsets = at<int32_t>(workspace, w.offsets);
  int32_t* perm = at<int32_t>(workspace, w.perm);
  int32_t* bmap = at<int32_t>(workspace, w.bmap);
  int32_t* ntiles = at<int32_t>(workspace, w.ntiles);
  uint16_t* h = at<uint16_t>(workspace, w.h);
  uint16_t* hsh = at<uint16_t>(workspace, w.hsh);
  const int E = d->n_experts, k = d->top_k;
  const int mt = moe_max_tiles(T, k, E, kBM);
  // shared-expert chunks of kBM rows go first in the same launches as the routed tiles
  int32_t* trows = at<int32_t>(workspace, w.trows);
  const GemmTiles tl{perm, offsets, bmap, ntiles, mt, kBM, static_cast<int32_t>(div_up(T, kBM)), trows};

  // router output: final logits (one K split) or per-split partial sums that top-k adds up in order
  const int S = w.splits;
  float* rout = S > 1 ? at<float>(workspace, w.rparts) : logits;
  float* sout = S > 1 ? at<float>(workspace, w.sparts) : s_logit;
  if (run(MOE_STAGE_ROUTER) &&
      (st = hip_check(launch_router_gemm(x, L->router_w3, L->router_bias, L->shared_gate_w, T, d->hidden, E, S, rout,
                                         sout, s),
                      "router gemm")))
    return st;
  if (run(MOE_STAGE_TOPK) &&
      // with K splits top-k forms the final logits; they are stored only when
      // the caller asked for them (nothing downstream reads them)
      (st = hip_check(launch_topk(rout, sout, S, L->router_bias, T, E, k, S > 1 ? logits_out : logits, s_logit, ids,
                                  wts, gate, tilehist, s),
                      "top-k")))
    return st;
  if (run(MOE_STAGE_GROUP) &&
      (st = hip_check(launch_group(ids, tilehist, at<int32_t>(workspace, w.tilebase), T, k, E, kBM, counts, offsets,
                                   perm, at<int32_t>(workspace, w.inv), bmap, mt, ntiles, trows, err, s),
                      "grouping")))
    return st;
  if (run(MOE_STAGE_GATE_UP) &&
      (st = hip_check(launch_gemm_swiglu(*d, L->gate_up, &L->sh_gate_up, x, true, tl, T, h, hsh, s),
                      "gate/up gemm")))
    return st;
  // slots are stored unweighted; the combine applies routing weights and the gate
  if (run(MOE_STAGE_DOWN) &&
      (st = hip_check(launch_gemm_slots(*d, L->down, &L->sh_down, h, hsh, tl, T, slots, sexp, s), "down gemm")))
    return st;
  if (run(MOE_STAGE_COMBINE) &&
      (st = hip_check(launch_combine(slots, sexp, wts, gate, y, T, d->hidden, k, s), "combine")))
    return st;
  return MOE_OK;
}

moe_status moe_forward(const moe_dims* d, const moe_layer* L, const uint16_t* x, int32_t T, uint16_t* y,
                       float* logits_out, int32_t* ids_out, float* w_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return moe_forward_stages(d, L, x, T, y, logits_out, ids_out, w_out, workspace, workspace_bytes, MOE_STAGE_ROUTER,
                            MOE_STAGE_COMBINE, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation entry point

// Scratch of moe_forward_noalloc: one whole moe_forward workspace, a device
// global, so that the call needs no allocation.  Each device the library runs
// on holds its own copy until the process ends; device globals start
// zero-filled, which the fused path's hand-over words need before their first
// call.  In host code `scratch` names a host-side stand-in: its device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

moe_status scratch_address(void** out) {
  int dev = 0;
  moe_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if ((st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))) return st;
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const moe_dims* d, const moe_layer* L, const uint16_t* x, int32_t T, uint16_t* y,
                               float* logits_out, int32_t* ids_out, float* w_out, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  const size_t need = layout(*d, T).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "T=%d needs %zu bytes of scratch; moe_forward_noalloc holds %zu", T, need,
                static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return moe_forward_stages(d, L, x, T, y, logits_out, ids_out, w_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                            MOE_STAGE_ROUTER, MOE_STAGE_COMBINE, stream);
}

moe_status moe_host_block_map(const int32_t* counts, int32_t E, int32_t block_m, int32_t max_tiles, int32_t* offsets,
                              int32_t* block_map, int32_t* n_tiles) {
  if (!counts || !offsets || !block_map || !n_tiles) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (E < 1 || block_m < 1 || max_tiles < 0) return fail(MOE_ERR_INVALID_ARG, "E, block_m must be positive");
  int64_t off = 0, tiles = 0;
  for (int e = 0; e < E; ++e) {
    if (counts[e] < 0) return fail(MOE_ERR_INVALID_ARG, "counts[%d] = %d is negative", e, counts[e]);
    tiles += (counts[e] + block_m - 1) / block_m;
    off += counts[e];
    if (off > INT32_MAX) return fail(MOE_ERR_INVALID_ARG, "counts sum past 2^31");
  }
  if (tiles > max_tiles) return fail(MOE_ERR_INVALID_ARG, "max_tiles=%d < %lld tiles", max_tiles,
                                     static_cast<long long>(tiles));
  int32_t o = 0, t = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = o;
    for (int32_t r = 0; r < counts[e]; r += block_m, ++t) {
      block_map[2 * t] = e;
      block_map[2 * t + 1] = o + r;
    }
    o += counts[e];
  }
  offsets[E] = o;
  *n_tiles = t;
  for (int32_t i = t; i < max_tiles; ++i) block_map[2 * i] = block_map[2 * i + 1] = -1;
  return MOE_OK;
}

size_t moe_host_routing_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) || check_T(T)) return 0;
  const int E = d->n_experts;
  return 4 * (static_cast<size_t>(E) + E + 1 + 2 * static_cast<size_t>(moe_max_tiles(T, d->top_k, E, kBM)) + 1);
}

moe_status moe_forward_host_routing(const moe_dims* d, const moe_layer* L, const uint16_t* x, int32_t T,
                                    uint16_t* y, int32_t* ids_out, float* w_out, void* workspace,
                                    size_t workspace_bytes, void* host_buf, size_t host_bytes, void* stream) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if (T <= kDecMaxT && decode_supported(*d, T))
    return fail(MOE_ERR_UNSUPPORTED, "the host-routed variant covers the grouped path only (T=%d runs fused)", T);
  const size_t need = moe_host_routing_bytes(d, T);
  if (!host_buf || host_bytes < need) return fail(MOE_ERR_INVALID_ARG, "host buffer %zu < %zu bytes", host_bytes, need);
  // router and top-k exactly as in moe_forward (this also validates the rest)
  if ((st = moe_forward_stages(d, L, x, T, y, nullptr, ids_out, w_out, workspace, workspace_bytes, MOE_STAGE_ROUTER,
                               MOE_STAGE_TOPK, stream)))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws w = layout(*d, T);
  const int E = d->n_experts, k = d->top_k;
  const int mt = moe_max_tiles(T, k, E, kBM);
  const int32_t* ids = ids_out ? ids_out : at<int32_t>(workspace, w.ids);
  int32_t* counts = at<int32_t>(workspace, w.counts);
  int32_t* offsets = at<int32_t>(workspace, w.offsets);
  int32_t* bmap = at<int32_t>(workspace, w.bmap);
  int32_t* ntiles = at<int32_t>(workspace, w.ntiles);
  int32_t* tilebase = at<int32_t>(workspace, w.tilebase);
  int32_t* h_counts = static_cast<int32_t*>(host_buf);
  int32_t* h_offsets = h_counts + E;
  int32_t* h_bmap = h_offsets + E + 1;
  int32_t* h_ntiles = h_bmap + 2 * mt;
  // counts to the host, wait, offsets + block map on the host, back to the GPU
  if ((st = hip_check(launch_group_counts(at<int32_t>(workspace, w.tilehist), tilebase, T, E, counts, s),
                      "expert counts")) ||
      (st = hip_check(hipMemcpyAsync(h_counts, counts, 4 * E, hipMemcpyDeviceToHost, s), "counts to host")) ||
      (st = hip_check(hipStreamSynchronize(s), "stream synchronize")))
    return st;
  if ((st = moe_host_block_map(h_counts, E, kBM, mt, h_offsets, h_bmap, h_ntiles))) return st;
  if ((st = hip_check(hipMemcpyAsync(offsets, h_offsets, 4 * (E + 1), hipMemcpyHostToDevice, s), "offsets")) ||
      (st = hip_check(hipMemcpyAsync(bmap, h_bmap, 8 * static_cast<size_t>(mt), hipMemcpyHostToDevice, s),
                      "block map")) ||
      (st = hip_check(hipMemcpyAsync(ntiles, h_ntiles, 4, hipMemcpyHostToDevice, s), "n_tiles")) ||
      (st = hip_check(launch_group_scatter(ids, counts, tilebase, T, k, E, kBM, offsets,
                                           at<int32_t>(workspace, w.perm), at<int32_t>(workspace, w.inv), bmap, mt,
                                           ntiles, false, at<int32_t>(workspace, w.trows),
                                           at<uint32_t>(workspace, 0), s),
                      "permutation")))
    return st;
  return moe_forward_stages(d, L, x, T, y, nullptr, ids_out, w_out, workspace, workspace_bytes, MOE_STAGE_GATE_UP,
                            MOE_STAGE_COMBINE, stream);
}

moe_status moe_fused_residency(const moe_dims* d, int32_t T, int32_t* needed, int32_t* resident) {
  moe_status st = check_dims(d);
  if (st) return st;
  if ((st = check_T(T))) return st;
  if (!needed || !resident) return fail(MOE_ERR_INVALID_ARG, "NULL output pointer");
  *needed = 0;
  *resident = 0;
  if (!(T <= kDecMaxT && decode_supported(*d, T)))
    return fail(MOE_ERR_UNSUPPORTED, "T=%d does not run the fused layer for these dims", T);
  int n = 0, r = 0;
  if ((st = hip_check(fused_residency(*d, T, &n, &r), "device query"))) return st;
  *needed = n;
  *resident = r;
  return MOE_OK;
}

moe_status moe_workspace_errors(void* workspace, size_t workspace_bytes, int32_t clear, int32_t* flags,
                                void* stream) {
  if (!workspace || workspace_bytes < kWsHeader) return fail(MOE_ERR_WORKSPACE, "workspace missing or too small");
  if (!flags) return fail(MOE_ERR_INVALID_ARG, "flags is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* word = at<uint32_t>(workspace, 0);
  uint32_t v = 0;
  moe_status st;
  if ((st = hip_check(hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, s), "error word to host")) ||
      (st = hip_check(hipStreamSynchronize(s), "stream synchronize")))
    return st;
  *flags = static_cast<int32_t>(v);
  if (clear) {
    hipLaunchKernelGGL(k_clear_word, dim3(1), dim3(1), 0, s, word);
    if ((st = hip_check(hipGetLastError(), "clear error word")) ||
        (st = hip_check(hipStreamSynchronize(s), "stream synchronize")))
      return st;
  }
  return MOE_OK;
}

// ------------------------------------------------------------------ grouped-query decode attention

namespace {
moe_status check_gqa(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S) {
  if (B < 1 || B > 4096 || Hq < 1 || Hkv < 1 || S < 1 || S > (1 << 22))
    return fail(MOE_ERR_INVALID_ARG, "gqa: need 1 <= B <= 4096, Hq, Hkv >= 1, 1 <= S <= 2^22");
  if (Hq % Hkv) return fail(MOE_ERR_INVALID_ARG, "gqa: Hq %% Hkv != 0");
  if (Hq / Hkv > 8 || Hq > 1024) return fail(MOE_ERR_UNSUPPORTED, "gqa: at most 8 query heads per key/value head");
  if (D != 64 && D != 128 && D != 256) return fail(MOE_ERR_UNSUPPORTED, "gqa: head_dim must be 64, 128 or 256");
  return MOE_OK;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

size_t moe_gqa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S) {
  if (check_gqa(B, Hq, Hkv, D, S)) return 0;
  return gqa_workspace_bytes(B, Hq, Hkv, S, D);
}

moe_status moe_gqa_decode_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                    const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                                    float scale, int32_t pack_heads, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  moe_status st = check_gqa(B, Hq, Hkv, D, S);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !seq_lens || !out) return fail(MOE_ERR_INVALID_ARG, "gqa: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(MOE_ERR_INVALID_ARG, "gqa: caches not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(q) & 3u) return fail(MOE_ERR_INVALID_ARG, "gqa: q not 4-byte aligned");
  if (pack_heads != 0 && pack_heads != 1) return fail(MOE_ERR_INVALID_ARG, "gqa: pack_heads must be 0 or 1");
  if (!workspace || !aligned16(workspace) || workspace_bytes < gqa_workspace_bytes(B, Hq, Hkv, S, D))
    return fail(MOE_ERR_WORKSPACE, "gqa: workspace missing, unaligned or smaller than moe_gqa_decode_workspace_bytes");
  return hip_check(launch_gqa_decode(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S, scale, pack_heads == 1, out,
                                     workspace, static_cast<hipStream_t>(stream)),
                   "gqa decode");
}

}  // extern "C"
