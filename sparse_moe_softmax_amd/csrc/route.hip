// Router: logits = x . W_r^T (+ bias), shared-gate logit, top-k selection with
// renormalised softmax weights, and the per-tile expert histogram that the
// grouping step scans.  Each token is scored against all 256 routed experts,
// the best 8 are kept, and the shared expert runs for every token (Lily page,
// section "The architecture that forces the issue: MoE plus Gated DeltaNet").
#include "topk.hpp"

namespace moe {

// ------------------------------------------------------------------ prepack

// w = hi + mid + lo exactly, each a bfloat16 holding the next 8 significant
// bits of w (truncation split; exact for |w| >= 2^-100 and for 0).
__global__ void k_prepack_router(const float* __restrict__ w, uint16_t* __restrict__ w3, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = w[i];
  const uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mb);
  w3[i] = static_cast<uint16_t>(hb >> 16);
  w3[n + i] = static_cast<uint16_t>(mb >> 16);
  w3[2 * n + i] = static_cast<uint16_t>(__float_as_uint(r2) >> 16);
}

hipError_t launch_prepack_router(const float* w, uint16_t* w3, int E, int H, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(E) * H;
  hipLaunchKernelGGL(k_prepack_router, dim3(static_cast<unsigned>(div_up(n, 256))), dim3(256), 0, s, w, w3, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router GEMM (T > 1)

// Tile of 64 tokens x 64 experts over one K range (K may be split over
// gridDim.z workgroups so that small T still fills the chip).  Per 64-wide K
// block, direct-to-LDS loads bring the bf16 x tile (8 KB), the three bf16
// weight planes of the 64 experts (24 KB) and the 64 shared-gate weights into
// a ring of kRtStages stages, refilled kRtStages-1 blocks ahead (the same
// explicit-vmcnt scheme as the grouped GEMM; rows XOR-swizzled by a_chunk).
// Two stages (66 KB) let two workgroups share a CU: the loop is bound by its
// per-block chain of waits, so a second workgroup covers it better than a
// deeper ring (four stages, one workgroup per CU, was 36 µs against 26 µs at
// T = 4096).
// Wave w owns experts [16w, 16w + 16) of the tile for all 64 tokens (4 MFMA
// row sub-tiles of v_mfma_f32_16x16x32_bf16).  Within a K block the lane group
// q = lane/16 covers K offsets [16q, 16q+16): k-step s of a lane holds offsets
// 16q + 8s .. +7 for both operands (a consistent permutation of K).
// Workgroups of the first expert tile also form the shared-gate dot product
// on the vector ALUs from the staged x tile.
// One split: logits (+ bias) and s_logit are final.  Several: partial sums
// part[z][T][E], s_part[z][T] without bias, summed in z order by k_topk.
constexpr int kRtM = 64;
constexpr int kRtN = 64;
constexpr int kRtStages = 2;
constexpr int kRtX = kRtM * 128;                  // x tile
constexpr int kRtW = 3 * kRtN * 128;              // weight planes
constexpr int kRtS = 4 * 256;                     // shared-gate weights (one copy per wave)
constexpr int kRtStage = kRtX + kRtW + kRtS;
constexpr int kRtDma = 2 + 6 + 1;                 // loads per wave per stage
constexpr int kMaxSplits = 8;                     // K splits at most

__global__ __launch_bounds__(256) void k_router_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w3,
                                                     const float* __restrict__ bias, const float* __restrict__ wsg,
                                                     int T, int H, int E, int kbs, float* __restrict__ out,
                                                     float* __restrict__ s_out) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRtStages * kRtStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int col = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * kRtM;
  const int rows = min(kRtM, T - t0);
  const int e0 = blockIdx.y * kRtN;
  const int z = blockIdx.z;
  const int splits = gridDim.z;
  const int kb0 = z * kbs;
  const bool do_s = blockIdx.y == 0 && s_out != nullptr;

  // per-lane load offsets (bytes); rows past T or E re-read the last valid row
  uint32_t xoff[2], woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (wave * 2 + j) * 8 + (lane >> 3);
    const int p = lane & 7;
    int c = 0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      if (a_chunk(r, cc) == p) c = cc;
    xoff[j] = (static_cast<uint32_t>(t0 + min(r, rows - 1)) * H + kb0 * 64 + c * 8) * 2;
    woff[j] = (static_cast<uint32_t>(min(e0 + r, E - 1)) * H + kb0 * 64 + c * 8) * 2;
  }
  const uint32_t plane_bytes = static_cast<uint32_t>(E) * H * 2;
  const i32x4 xr = buffer_rsrc(x), wr = buffer_rsrc(w3), sr = buffer_rsrc(wsg);
  const uint32_t soff = (kb0 * 64 + lane) * 4;
  const uint32_t ring_s = lds_addr(ring);

  auto issue = [&](int kb) {
    const uint32_t st = ring_s + (kb % kRtStages) * kRtStage;
    const uint32_t ko = kb * 128;
#pragma unroll
    for (int j = 0; j < 2; ++j) bdma16(xr, xoff[j], ko, st + (wave_s * 2 + j) * 1024);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) bdma16(wr, woff[j] + p * plane_bytes, ko, st + kRtX + p * 8192 + (wave_s * 2 + j) * 1024);
    bdma4(sr, soff, kb * 256, st + kRtX + kRtW + wave_s * 256);
  };

  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float s_acc = 0.f;
  const int s_tok = tid >> 2, s_q = tid & 3;

#pragma unroll
  for (int st = 0; st < kRtStages - 1; ++st)
    if (st < kbs) issue(st);
  for (int kb = 0; kb < kbs; ++kb) {
    // issued so far: stages 0 .. min(kb + kRtStages - 2, kbs - 1); wait for stage kb
    wait_stages<kRtDma, kRtStages - 2>(min(kRtStages - 2, kbs - 1 - kb));
    __builtin_amdgcn_s_barrier();  // stage kb landed for every wave; stage kb-1 consumed
    if (kb + kRtStages - 1 < kbs) issue(kb + kRtStages - 1);
    const unsigned char* st = ring + (kb % kRtStages) * kRtStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[4], b[3];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = m * 16 + col;
        a[m] = *reinterpret_cast<const bf16x8*>(st + r * 128 + (a_chunk(r, 2 * q + ks) << 4));
      }
      const int er = wave * 16 + col;
#pragma unroll
      for (int p = 0; p < 3; ++p)
        b[p] = *reinterpret_cast<const bf16x8*>(st + kRtX + p * 8192 + er * 128 + (a_chunk(er, 2 * q + ks) << 4));
#pragma unroll
      for (int p = 2; p >= 0; --p)   // planes lo, mid, hi
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = mfma16(a[m], b[p], acc[m]);
    }
    if (do_s) {
      const float* wsl = reinterpret_cast<const float*>(st + kRtX + kRtW);   // wave 0's copy
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * s_q + h;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(st + s_tok * 128 + (a_chunk(s_tok, c) << 4));
#pragma unroll
        for (int i = 0; i < 8; ++i) s_acc = __builtin_fmaf(static_cast<float>(v[i]), wsl[c * 8 + i], s_acc);
      }
    }
  }

  const int e = e0 + wave * 16 + col;
  if (e < E) {
    const bool last = splits == 1;
    const float b = (last && bias) ? bias[e] : 0.f;
    float* o = out + static_cast<int64_t>(z) * T * E;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + q * 4 + i;
        if (r < rows) o[static_cast<int64_t>(t0 + r) * E + e] = acc[m][i] + b;
      }
  }
  if (do_s) {
    s_acc += __shfl_xor(s_acc, 1);
    s_acc += __shfl_xor(s_acc, 2);
    if (s_q == 0 && s_tok < rows) s_out[static_cast<int64_t>(z) * T + t0 + s_tok] = s_acc;
  }
}

// Wide form for large T: tiles of 128 tokens x 128 experts, 32-wide K blocks,
// so that each weight plane row staged in LDS serves twice the tokens and each
// x row twice the experts (half the bytes per flop of the 64 x 64 form).
// 64-byte rows, 16-byte chunk c of row r stored at position c ^ ((r >> 2) & 3):
// 16 consecutive rows read at one chunk hit 16 distinct bank groups.  Wave w
// owns experts [32w, 32w + 32) for all 128 tokens (8 x 2 sub-tiles of
// v_mfma_f32_16x16x32_bf16); lane group q = lane/16 covers K offsets
// [8q, 8q + 8) of the block for both operands.  Shared gate, splits and
// outputs as in the 64 x 64 form.
constexpr int kRwM = 128;
constexpr int kRwN = 128;
constexpr int kRwStages = 2;   // 66 KB: two workgroups per CU, as for the 64 x 64 form
constexpr int kRwX = kRwM * 64;                   // x tile: 128 rows x 32 K
constexpr int kRwW = 3 * kRwN * 64;               // weight planes
constexpr int kRwS = 4 * 256;                     // shared-gate weights (one copy per wave)
constexpr int kRwStage = kRwX + kRwW + kRwS;
constexpr int kRwDma = 2 + 6 + 1;                 // loads per wave per stage

__device__ inline int rw_pos(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ __launch_bounds__(256) void k_router_gemm_wide(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w3,
                                                          const float* __restrict__ bias,
                                                          const float* __restrict__ wsg, int T, int H, int E,
                                                          int kbs, float* __restrict__ out,
                                                          float* __restrict__ s_out) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRwStages * kRwStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int col = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * kRwM;
  const int rows = min(kRwM, T - t0);
  const int e0 = blockIdx.y * kRwN;
  const int z = blockIdx.z;
  const int splits = gridDim.z;
  const int kb0 = z * kbs;                         // first 32-wide K block of this split
  const bool do_s = blockIdx.y == 0 && s_out != nullptr;

  // per-lane load offsets (bytes): instruction j of wave w fills rows
  // (2w + j) * 16 + lane/4, physical chunk lane % 4; rows past T or E re-read
  // the last valid row
  uint32_t xoff[2], woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (wave * 2 + j) * 16 + (lane >> 2);
    const int c = rw_pos(r, lane & 3);             // the logical chunk stored at this position
    xoff[j] = (static_cast<uint32_t>(t0 + min(r, rows - 1)) * H + kb0 * 32 + c * 8) * 2;
    woff[j] = (static_cast<uint32_t>(min(e0 + r, E - 1)) * H + kb0 * 32 + c * 8) * 2;
  }
  const uint32_t plane_bytes = static_cast<uint32_t>(E) * H * 2;
  const i32x4 xr = buffer_rsrc(x), wr = buffer_rsrc(w3), sr = buffer_rsrc(wsg);
  const uint32_t soff = (kb0 * 32 + (lane & 31)) * 4;   // 32 weights per block, duplicated in the upper lanes
  const uint32_t ring_s = lds_addr(ring);

  auto issue = [&](int kb) {
    const uint32_t st = ring_s + (kb % kRwStages) * kRwStage;
    const uint32_t ko = kb * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j) bdma16(xr, xoff[j], ko, st + (wave_s * 2 + j) * 1024);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bdma16(wr, woff[j] + p * plane_bytes, ko, st + kRwX + p * 8192 + (wave_s * 2 + j) * 1024);
    bdma4(sr, soff, kb * 128, st + kRwX + kRwW + wave_s * 256);
  };

  f32x4 acc[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float s_acc = 0.f;
  const int s_tok = tid >> 1, s_h = tid & 1;

#pragma unroll
  for (int st = 0; st < kRwStages - 1; ++st)
    if (st < kbs) issue(st);
  for (int kb = 0; kb < kbs; ++kb) {
    // issued so far: stages 0 .. min(kb + kRwStages - 2, kbs - 1); wait for stage kb
    wait_stages<kRwDma, kRwStages - 2>(min(kRwStages - 2, kbs - 1 - kb));
    __builtin_amdgcn_s_barrier();  // stage kb landed for every wave; stage kb-1 consumed
    if (kb + kRwStages - 1 < kbs) issue(kb + kRwStages - 1);
    const unsigned char* st = ring + (kb % kRwStages) * kRwStage;
    bf16x8 a[8], b[2][3];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int r = m * 16 + col;
      a[m] = *reinterpret_cast<const bf16x8*>(st + r * 64 + (rw_pos(r, q) << 4));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int er = wave * 32 + j * 16 + col;
#pragma unroll
      for (int p = 0; p < 3; ++p)
        b[j][p] = *reinterpret_cast<const bf16x8*>(st + kRwX + p * 8192 + er * 64 + (rw_pos(er, q) << 4));
    }
#pragma unroll
    for (int p = 2; p >= 0; --p)   // planes lo, mid, hi
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m][j] = mfma16(a[m], b[j][p], acc[m][j]);
    if (do_s) {
      const float* wsl = reinterpret_cast<const float*>(st + kRwX + kRwW);   // wave 0's copy
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * s_h + h;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(st + s_tok * 64 + (rw_pos(s_tok, c) << 4));
#pragma unroll
        for (int i = 0; i < 8; ++i) s_acc = __builtin_fmaf(static_cast<float>(v[i]), wsl[c * 8 + i], s_acc);
      }
    }
  }

  const bool last = splits == 1;
  float* o = out + static_cast<int64_t>(z) * T * E;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + wave * 32 + j * 16 + col;
    if (e < E) {
      const float b = (last && bias) ? bias[e] : 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m * 16 + q * 4 + i;
          if (r < rows) o[static_cast<int64_t>(t0 + r) * E + e] = acc[m][j][i] + b;
        }
    }
  }
  if (do_s) {
    s_acc += __shfl_xor(s_acc, 1);
    if (s_h == 0 && s_tok < rows) s_out[static_cast<int64_t>(z) * T + t0 + s_tok] = s_acc;
  }
}

// Tile form and K splits for T tokens: the wide form where its tiles alone
// fill the chip (256 workgroups), else 64 x 64 tiles; either split over K as
// far as needed (at most kMaxSplits) to give every CU two workgroups.
struct RouterPlan {
  bool wide;
  int splits;
};
static RouterPlan router_plan(int T, int H, int E) {
  const int64_t wide_tiles = div_up(T, kRwM) * div_up(E, kRwN);
  if (wide_tiles >= 256) {
    int ws = static_cast<int>(div_up(512, wide_tiles));
    while (ws > 1 && (H / 32) % ws) --ws;
    return {true, ws};
  }
  const int64_t tiles = div_up(T, kRtM) * div_up(E, kRtN);
  const int kg = H / 64;
  int want = static_cast<int>(div_up(512, tiles));
  want = want < 1 ? 1 : (want > kMaxSplits ? kMaxSplits : want);
  while (want > 1 && kg % want) --want;
  return {false, want};
}

int router_splits(int T, int H, int E) { return router_plan(T, H, E).splits; }

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w3, const float* bias, const float* wsg, int T,
                              int H, int E, int splits, float* out, float* s_out, hipStream_t s) {
  const RouterPlan plan = router_plan(T, H, E);
  const float* wsg_src = wsg ? wsg : reinterpret_cast<const float*>(w3);   // loaded but unused without s_out
  if (plan.wide && splits == plan.splits) {
    dim3 grid(static_cast<unsigned>(div_up(T, kRwM)), static_cast<unsigned>(div_up(E, kRwN)),
              static_cast<unsigned>(splits));
    hipLaunchKernelGGL(k_router_gemm_wide, grid, dim3(256), 0, s, x, w3, bias, wsg_src, T, H, E, H / 32 / splits,
                       out, wsg ? s_out : nullptr);
  } else {
    dim3 grid(static_cast<unsigned>(div_up(T, kRtM)), static_cast<unsigned>(div_up(E, kRtN)),
              static_cast<unsigned>(splits));
    hipLaunchKernelGGL(k_router_gemm, grid, dim3(256), 0, s, x, w3, bias, wsg_src, T, H, E, H / 64 / splits, out,
                       wsg ? s_out : nullptr);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ router GEMV (T == 1 path)

// One wave per weight row (rows 0..E-1 = experts, row E = shared gate), fp32
// dot products with coalesced float4 weight loads.
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ bias, const float* __restrict__ wsg,
                                                     int T, int H, int E, float* __restrict__ logits,
                                                     float* __restrict__ s_logit) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r > E || (r == E && !s_logit)) return;
  const float* wr = (r < E) ? w + static_cast<int64_t>(r) * H : wsg;
  for (int t = 0; t < T; ++t) {
    const uint16_t* xr = x + static_cast<int64_t>(t) * H;
    float acc = 0.f;
    for (int k = lane * 4; k < H; k += 256) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + k);
      const uint2 xv = *reinterpret_cast<const uint2*>(xr + k);
      acc = __builtin_fmaf(__uint_as_float(xv.x << 16), wv.x, acc);
      acc = __builtin_fmaf(__uint_as_float(xv.x & 0xFFFF0000u), wv.y, acc);
      acc = __builtin_fmaf(__uint_as_float(xv.y << 16), wv.z, acc);
      acc = __builtin_fmaf(__uint_as_float(xv.y & 0xFFFF0000u), wv.w, acc);
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      if (r < E)
        logits[static_cast<int64_t>(t) * E + r] = acc + (bias ? bias[r] : 0.f);
      else
        s_logit[t] = acc;
    }
  }
}

hipError_t launch_router_gemv(const uint16_t* x, const float* w, const float* bias, const float* wsg, int T, int H,
                              int E, float* logits, float* s_logit, hipStream_t s) {
  hipLaunchKernelGGL(k_router_gemv, dim3(static_cast<unsigned>(div_up(E + 1, 4))), dim3(256), 0, s, x, w, bias, wsg,
                     T, H, E, logits, s_logit);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k

// One block = one routing tile of kTopkTile tokens, one wave per token; lane l
// holds experts l, l + 64, l + 128, l + 192 (coalesced loads).  With several
// router splits the logits are first summed over the splits in order (plus the
// bias) and written out.  Optionally counts the tile's expert histogram.
constexpr int kTopkThreads = kTopkTile * 64;

template <int K>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ parts,
                                                       const float* __restrict__ s_parts, int splits,
                                                       const float* __restrict__ bias, int T, int E, int k,
                                                       float* __restrict__ logits_out, float* __restrict__ s_out,
                                                       int32_t* __restrict__ ids, float* __restrict__ wts,
                                                       float* __restrict__ gate, int32_t* __restrict__ tilehist) {
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = blockIdx.x * kTopkTile + (tid >> 6);
  if (tilehist) {
    for (int e = tid; e < E; e += kTopkThreads) hist[e] = 0;
    __syncthreads();
  }
  if (t < T) {
    const int64_t TE = static_cast<int64_t>(T) * E;
    const int64_t o = static_cast<int64_t>(t) * E;
    // all partial sums are loaded first (one round trip), then added in split order
    float p[kMaxSplits][4];
#pragma unroll
    for (int zz = 0; zz < kMaxSplits; ++zz)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (zz < splits && lane + 64 * i < E) p[zz][i] = parts[zz * TE + o + lane + 64 * i];
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      v[i] = 0.f;
      if (e < E) {
        float l = p[0][i];
#pragma unroll
        for (int zz = 1; zz < kMaxSplits; ++zz)
          if (zz < splits) l += p[zz][i];
        if (splits > 1) {
          if (bias) l += bias[e];
          if (logits_out) logits_out[o + e] = l;
        }
        v[i] = l;
      }
    }
    int my_e = 0;
    float my_w = 0.f;
    if constexpr (K > 0) {
      // lane r < K holds slot r; its weight exp(l_r - l_0) / sum, the sum
      // taken in slot order (the same values as topk_weights)
      float my_v;
      topk_wave64_fixed<K>(v, E, my_e, my_v);
      const float top0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
      const float ex = expf(my_v - top0);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < K; ++r) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), r));
      my_w = ex * (1.0f / sum);
    } else {
      int te[16];
      float tv[16], w[16];
      topk_wave64_regs(v, E, k, te, tv);
      topk_weights(k, tv, w);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r == lane) {
          my_e = te[r];
          my_w = w[r];
        }
    }
    if (lane < k) {
      ids[static_cast<int64_t>(t) * k + lane] = my_e;
      wts[static_cast<int64_t>(t) * k + lane] = my_w;
      if (tilehist) atomicAdd(&hist[my_e], 1);
    }
    if (s_parts && lane == 0) {
      float sp[kMaxSplits];
#pragma unroll
      for (int zz = 0; zz < kMaxSplits; ++zz)
        if (zz < splits) sp[zz] = s_parts[static_cast<int64_t>(zz) * T + t];
      float sl = sp[0];
#pragma unroll
      for (int zz = 1; zz < kMaxSplits; ++zz)
        if (zz < splits) sl += sp[zz];
      if (splits > 1 && s_out) s_out[t] = sl;
      if (gate) gate[t] = sigmoidf_(sl);
    }
  }
  if (tilehist) {
    __syncthreads();
    for (int e = tid; e < E; e += kTopkThreads) tilehist[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
  }
}

hipError_t launch_topk(const float* parts, const float* s_parts, int splits, const float* bias, int T, int E, int k,
                       float* logits_out, float* s_out, int32_t* ids, float* wts, float* gate, int32_t* tilehist,
                       hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(div_up(T, kTopkTile)));
  if (k == 8)
    hipLaunchKernelGGL(k_topk<8>, grid, dim3(kTopkThreads), 0, s, parts, s_parts, splits, bias, T, E, k, logits_out,
                       s_out, ids, wts, gate, tilehist);
  else
    hipLaunchKernelGGL(k_topk<0>, grid, dim3(kTopkThreads), 0, s, parts, s_parts, splits, bias, T, E, k, logits_out,
                       s_out, ids, wts, gate, tilehist);
  return hipGetLastError();
}

}  // namespace moe
