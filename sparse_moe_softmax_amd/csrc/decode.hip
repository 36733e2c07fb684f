// Batch-1 decode path of the MoE layer.  With one token per step every weight
// is used once, so the work is matrix-vector, limited by memory bandwidth, and
// the pages assign it to the vector ALUs rather than the matrix units (Lily
// page, section "Why Apple Silicon isn't just a smaller datacenter GPU"); chains
// of kernels are fused so that intermediates stay on chip (Inside Lily page,
// section "Performance Gains and Workload Patterns").
//
// Three launches per layer:
//   1. router GEMV (fp32 weights)                      -> logits, shared-gate logit
//   2. per (slot, 16 h-columns): top-k recomputed from the logits in every
//      block (no extra launch), gate/up GEMV of the slot's expert with the
//      int4 rows dequantised in registers, SwiGLU    -> h [k+1][ldh] bf16
//   3. per 16 output rows: down GEMV of all k+1 slots and the weighted combine
//      in slot order, shared expert last              -> y bf16
// No atomics: the output is bitwise reproducible.
#include "internal.hpp"

namespace moe {

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Dot product of 32 consecutive int4 weights of one quantisation group (one
// uint4 of codes) with 32 bf16 activations (four uint4).
__device__ inline float dot32(const uint4& codes, const DqConst& dc, const uint4 (&xv)[4], float acc) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = dequant8(cw[i], dc.s24, dc.s20, dc.bias);
    acc = dot2(w.x, xv[i].x, acc);
    acc = dot2(w.y, xv[i].y, acc);
    acc = dot2(w.z, xv[i].z, acc);
    acc = dot2(w.w, xv[i].w, acc);
  }
  return acc;
}

struct DecArgs {
  moe_q4 gu, dn, sgu, sdn;
  int H, I, Is, E, k;
  const uint16_t* x;       // [H] bf16
  const float* logits;     // [E]
  const float* s_logit;    // [1]
  int32_t* ids;            // [k] written by block (0, 0) of the gate/up kernel
  float* wts;              // [k]
  float* gate;             // [1]
  uint16_t* h;             // [k+1][ldh] bf16
  int ldh;
  uint16_t* y;             // [H] bf16
};

// grid: x = ceil(max(I, Is) / 16) column chunks, y = k + 1 slots (slot k = shared).
// Wave w computes h columns [16 bx + 4w, +4): 4 gate rows and the 4 matching up rows.
__global__ __launch_bounds__(256) void k_dec_gateup(DecArgs a) {
  __shared__ int s_e[16];
  __shared__ float s_w[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slot = blockIdx.y;
  const bool shared = slot == a.k;
  if (!shared) {
    if (tid < 16) {
      int te[16];
      float tv[16], w[16];
      topk16(a.logits, a.E, a.k, tid, te, tv);
      topk_weights(a.k, tv, w);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r == tid && r < a.k) {
          s_e[r] = te[r];
          s_w[r] = w[r];
        }
    }
    __syncthreads();
    if (blockIdx.x == 0 && slot == 0 && tid < a.k) {
      a.ids[tid] = s_e[tid];
      a.wts[tid] = s_w[tid];
      if (tid == 0) a.gate[0] = sigmoidf_(a.s_logit[0]);
    }
  }
  const int Ih = shared ? a.Is : a.I;
  const int hc = blockIdx.x * 16 + wave * 4;
  if (hc >= Ih) return;
  const int64_t e = shared ? 0 : s_e[slot];
  const moe_q4 q = shared ? a.sgu : a.gu;
  const int H = a.H;
  const int64_t nrow = 2 * static_cast<int64_t>(Ih);
  const uint8_t* cb = q.codes + e * nrow * (H / 2);
  const uint16_t* sb = q.scales + e * nrow * (H / 64);
  const uint16_t* bb = q.biases + e * nrow * (H / 64);

  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
  // lane covers K = [32 lane + 2048 c, +32) for c = 0, 1, ...
  for (int k0 = lane * 32; k0 < H; k0 += 2048) {
    uint4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const uint4*>(a.x + k0 + 8 * i);
    uint4 cw[8];
    uint16_t sv[8], bv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t row = (r < 4) ? hc + r : Ih + hc + (r - 4);
      cw[r] = *reinterpret_cast<const uint4*>(cb + row * (H / 2) + k0 / 2);
      sv[r] = sb[row * (H / 64) + k0 / 64];
      bv[r] = bb[row * (H / 64) + k0 / 64];
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = dot32(cw[r], dq_const(sv[r], bv[r]), xv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[r] += __shfl_xor(acc[r], off);
  if (lane < 4) {
    float gt = acc[0], up = acc[4];
#pragma unroll
    for (int r = 1; r < 4; ++r)
      if (lane == r) {
        gt = acc[r];
        up = acc[r + 4];
      }
    const float h = gt / (1.0f + __expf(-gt)) * up;
    a.h[static_cast<int64_t>(slot) * a.ldh + hc + lane] = f32_to_bf16_bits(h);
  }
}

// grid: H / 16 blocks; wave w, lane group g = lane / 16 computes output row
// n = 16 bx + 4 w + g with 16 lanes sharing the K dimension.
__global__ __launch_bounds__(256) void k_dec_down(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int k = a.k;
  const int nh = (k + 1) * a.ldh;
  for (int i = tid * 8; i < nh; i += 256 * 8)
    *reinterpret_cast<uint4*>(hs + i) = *reinterpret_cast<const uint4*>(a.h + i);
  __syncthreads();
  const int n = blockIdx.x * 16 + wave * 4 + (lane >> 4);
  const int j = lane & 15;
  float y = 0.f;
  for (int slot = 0; slot <= k; ++slot) {
    const bool shared = slot == k;
    const int K = shared ? a.Is : a.I;
    const int64_t e = shared ? 0 : a.ids[slot];
    const moe_q4 q = shared ? a.sdn : a.dn;
    const uint8_t* crow = q.codes + (e * a.H + n) * (K / 2);
    const uint16_t* srow = q.scales + (e * a.H + n) * (K / 64);
    const uint16_t* brow = q.biases + (e * a.H + n) * (K / 64);
    float acc = 0.f;
    for (int k0 = j * 32; k0 < K; k0 += 512) {
      const uint4 cw = *reinterpret_cast<const uint4*>(crow + k0 / 2);
      uint4 hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hv[i] = *reinterpret_cast<const uint4*>(hs + slot * a.ldh + k0 + 8 * i);
      acc = dot32(cw, dq_const(srow[k0 / 64], brow[k0 / 64]), hv, acc);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    const float wgt = shared ? a.gate[0] : a.wts[slot];
    y += wgt * acc;
  }
  if (j == 0) a.y[n] = f32_to_bf16_bits(y);
}

hipError_t launch_decode_stage(const moe_dims& d, const moe_layer& L, const uint16_t* x, uint16_t* y,
                               const DecodePtrs& p, int stage, hipStream_t s) {
  if (stage == MOE_STAGE_ROUTER)
    return launch_router_gemv(x, L.router_w, L.router_bias, L.shared_gate_w, 1, d.hidden, d.n_experts, p.logits,
                              p.s_logit, s);
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return hipSuccess;
  DecArgs a{};
  a.gu = L.gate_up;
  a.dn = L.down;
  a.sgu = L.sh_gate_up;
  a.sdn = L.sh_down;
  a.H = d.hidden;
  a.I = d.inter;
  a.Is = d.shared_inter;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.x = x;
  a.logits = p.logits;
  a.s_logit = p.s_logit;
  a.ids = p.ids;
  a.wts = p.wts;
  a.gate = p.gate;
  a.h = p.h;
  a.ldh = static_cast<int>(div_up(max(d.inter, d.shared_inter), 8) * 8);
  a.y = y;
  if (stage == MOE_STAGE_GATE_UP) {
    const int wmax = max(d.inter, d.shared_inter);
    hipLaunchKernelGGL(k_dec_gateup, dim3(static_cast<unsigned>(div_up(wmax, 16)), d.top_k + 1), dim3(256), 0, s, a);
  } else {
    const size_t shbytes = static_cast<size_t>(d.top_k + 1) * a.ldh * 2;
    hipLaunchKernelGGL(k_dec_down, dim3(static_cast<unsigned>(d.hidden / 16)), dim3(256), shbytes, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
