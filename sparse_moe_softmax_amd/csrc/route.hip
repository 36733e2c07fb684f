// Router: logits = x . W_r^T (+ bias), shared-gate logit, top-k selection with
// renormalised softmax weights, and the per-tile expert histogram that the
// grouping step scans.  ("A router scores 256 expert subnetworks and picks 8,
// plus a shared expert that runs on every token regardless": Lily page,
// section "The architecture that forces the issue: MoE plus Gated DeltaNet".)
#include "internal.hpp"

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

// Tile of 64 tokens x 64 experts, K in blocks of 64.  Wave w owns experts
// [e0 + 16w, e0 + 16w + 16) for all 64 tokens (4 MFMA row sub-tiles).  The
// bf16 x tile is staged in LDS; the three weight planes come straight from
// global memory as MFMA B fragments.  Within a 64-wide K block the lane
// group q = lane/16 covers K offsets [16q, 16q+16): fragment s of a lane holds
// offsets 16q + 8s .. 16q + 8s + 7 for both operands (a consistent
// permutation of K, which leaves the dot products unchanged).
constexpr int kRtM = 64;
constexpr int kRtN = 64;
constexpr int kLdA = 64 + 8;  // padded LDS row (144 B) to spread banks

__global__ __launch_bounds__(256) void k_router_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w3,
                                                     const float* __restrict__ bias, const float* __restrict__ wsg,
                                                     int T, int H, int E, float* __restrict__ logits,
                                                     float* __restrict__ s_logit, float* __restrict__ y_zero) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kRtM * kLdA];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRtM;
  const int rows = min(kRtM, T - t0);
  const int e_w = blockIdx.y * kRtN + wave * 16;
  const bool active = e_w < E;
  const int col = lane & 15;
  const int q = lane >> 4;
  const bool do_s = (blockIdx.y == 0) && (s_logit != nullptr);

  // zero this block's share of the fp32 combine buffer (moe_forward only)
  if (y_zero) {
    const int ny = gridDim.y;
    const int cw = static_cast<int>(div_up(div_up(H, ny), 4) * 4);
    const int c0 = blockIdx.y * cw;
    const int c1 = min(H, c0 + cw);
    const int w4 = (c1 - c0) / 4;
    for (int i = tid; i < rows * w4; i += 256) {
      const int r = i / w4, c = c0 + 4 * (i % w4);
      *reinterpret_cast<float4*>(y_zero + static_cast<int64_t>(t0 + r) * H + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  f32x4 acc[4];
  for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float s_acc = 0.f;
  const int s_tok = tid >> 2, s_q = tid & 3;
  const int64_t plane = static_cast<int64_t>(E) * H;
  const uint16_t* wrow = w3 + static_cast<int64_t>(active ? e_w + col : 0) * H;

  for (int kb = 0; kb < H / 64; ++kb) {
    // stage x[t0 .. t0+63][kb*64 .. +63] into LDS: 512 chunks of 16 B
    for (int c = tid; c < kRtM * 8; c += 256) {
      const int r = c >> 3, c8 = c & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < rows) v = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t0 + r) * H + kb * 64 + c8 * 8);
      *reinterpret_cast<uint4*>(As + r * kLdA + c8 * 8) = v;
    }
    __syncthreads();
    if (active) {
      // planes in order lo, mid, hi
      for (int p = 2; p >= 0; --p) {
        const uint16_t* src = wrow + p * plane + kb * 64 + q * 16;
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(src);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(src + 8);
        for (int m = 0; m < 4; ++m) {
          const uint16_t* ap = As + (m * 16 + col) * kLdA + q * 16;
          const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ap);
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ap + 8);
          acc[m] = mfma16(a0, b0, acc[m]);
          acc[m] = mfma16(a1, b1, acc[m]);
        }
      }
    }
    if (do_s) {
      const uint16_t* ap = As + s_tok * kLdA + s_q * 16;
      const float* wp = wsg + kb * 64 + s_q * 16;
      for (int i = 0; i < 16; ++i) s_acc = __builtin_fmaf(bf16_to_f32(ap[i]), wp[i], s_acc);
    }
    __syncthreads();
  }

  if (active) {
    const float b = bias ? bias[e_w + col] : 0.f;
    for (int m = 0; m < 4; ++m) {
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + q * 4 + i;
        if (r < rows) logits[static_cast<int64_t>(t0 + r) * E + e_w + col] = acc[m][i] + b;
      }
    }
  }
  if (do_s) {
    s_acc += __shfl_xor(s_acc, 1);
    s_acc += __shfl_xor(s_acc, 2);
    if (s_q == 0 && s_tok < rows) s_logit[t0 + s_tok] = s_acc;
  }
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w3, const float* bias, const float* wsg, int T,
                              int H, int E, float* logits, float* s_logit, float* y_zero, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(div_up(T, kRtM)), static_cast<unsigned>(div_up(E, kRtN)));
  hipLaunchKernelGGL(k_router_gemm, grid, dim3(256), 0, s, x, w3, bias, wsg, T, H, E, logits, s_logit, y_zero);
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

// One block = one routing tile of 64 tokens; 16 groups of 16 lanes take 16
// tokens at a time.  Optionally counts the tile's expert histogram.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ s_logit,
                                              int T, int E, int k, int32_t* __restrict__ ids,
                                              float* __restrict__ wts, float* __restrict__ gate,
                                              int32_t* __restrict__ tilehist) {
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  const int grp = tid >> 4, j = tid & 15;
  if (tilehist) {
    for (int e = tid; e < E; e += 256) hist[e] = 0;
    __syncthreads();
  }
  for (int it = 0; it < kTopkTile / 16; ++it) {
    const int t = blockIdx.x * kTopkTile + it * 16 + grp;
    if (t < T) {
      int te[16];
      float tv[16], w[16];
      topk16(logits + static_cast<int64_t>(t) * E, E, k, j, te, tv);
      topk_weights(k, tv, w);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r < k && r == j) {
          ids[static_cast<int64_t>(t) * k + r] = te[r];
          wts[static_cast<int64_t>(t) * k + r] = w[r];
          if (tilehist) atomicAdd(&hist[te[r]], 1);
        }
      }
      if (gate && s_logit && j == 0) gate[t] = sigmoidf_(s_logit[t]);
    }
  }
  if (tilehist) {
    __syncthreads();
    for (int e = tid; e < E; e += 256) tilehist[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
  }
}

hipError_t launch_topk(const float* logits, const float* s_logit, int T, int E, int k, int32_t* ids, float* wts,
                       float* gate, int32_t* tilehist, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3(static_cast<unsigned>(div_up(T, kTopkTile))), dim3(256), 0, s, logits, s_logit, T,
                     E, k, ids, wts, gate, tilehist);
  return hipGetLastError();
}

}  // namespace moe
