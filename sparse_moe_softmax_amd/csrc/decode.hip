// Batch-1 decode path of the MoE layer.  With one token per step every weight
// is used once, so the work is matrix-vector, limited by memory bandwidth, and
// the pages assign it to the vector ALUs rather than the matrix units (Lily
// page, section "Why Apple Silicon isn't just a smaller datacenter GPU"); chains
// of kernels are fused so that intermediates stay on chip (Inside Lily page,
// section "Performance Gains and Workload Patterns").
//
// The whole layer is one launch of kDecBlocks workgroups of 8 waves, all
// resident at once:
//   A. issue the loads that need no routing decision: this block's router
//      row(s), the shared expert's gate/up rows of this wave's column pair and
//      its down rows for this wave's output row;
//   B. router dot products (fp32 weights)              -> logit words
//   C. shared expert SwiGLU column pair                 -> h words of slot k
//   D. every block polls the logit words until all carry this call's tag and
//      recomputes top-k itself (one wave, lower expert index on ties), so the
//      routing decision needs no second round trip;
//   E. issue the routed experts' gate/up rows of this wave's (slot, column
//      pair) task and their down rows for this wave's output row;
//   F. routed SwiGLU column pairs                       -> h words of slot j
//   G. poll the h words; down GEMV over the k+1 slots with the weighted
//      combine in registers, slot order, shared expert last -> y (bf16).
// Int4 rows are dequantised in registers exactly as in the grouped GEMM
// (bf16 of the exact fp32 c*s + b) and multiplied with v_dot2_f32_bf16.
// No atomics on data: y is bitwise reproducible.
//
// Hand-over between workgroups: every value one block passes to others (a
// logit, two h values) travels in a 64-bit word whose high half is the tag of
// the call (its number + 1, modulo 2^32), written and read with agent-scope
// atomic stores and loads, which stay coherent across the XCDs' separate L2
// caches.  A consumer reads the words it needs until all carry the current
// tag, so one read gives both "ready" and the value: no counters, no
// read-modify-write atomics, no cache write-back or invalidate.  Each block
// keeps the number of calls it has completed in its own word of the
// workspace; all blocks finish every call, so they agree on it.  The
// workgroups of one launch are all resident (kDecBlocks <= CUs, one block fits
// a CU), so every wait ends; a wait that exceeds kSpinLimit polls sets the
// timeout word and carries on, so a launch always completes.
#include "internal.hpp"

namespace moe {

constexpr int kDecBlocks = 256;
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// 8 int4 weights of one group (one dword of codes) dotted with 8 bf16 (uint4).
__device__ inline float dot8(uint32_t codes, const DqConst& dc, const uint4& xv, float acc) {
  const uint4 w = dequant8(codes, dc.s24, dc.s20, dc.bias);
  acc = dot2(w.x, xv.x, acc);
  acc = dot2(w.y, xv.y, acc);
  acc = dot2(w.z, xv.z, acc);
  acc = dot2(w.w, xv.w, acc);
  return acc;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Workspace words of the T == 1 path (zero before the first call).
struct DecSync {
  uint32_t gen[kDecBlocks];   // calls completed, per block
  uint32_t timeout;
  uint32_t pad[63];
  uint64_t words[1];          // logit words [E + 1], then h words [k + 1][ldh / 2]
};

struct DecArgs {
  moe_q4 gu, dn, sgu, sdn;
  const float* router_w;   // [E][H]
  const float* router_bias;
  const float* wsg;        // [H]
  int H, I, Is, E, k;
  const uint16_t* x;       // [H] bf16
  float* logits;           // [E]
  float* s_logit;          // [1]
  int32_t* ids;            // [k]
  float* wts;              // [k]
  float* gate;             // [1]
  int ldh;                 // h row stride (multiple of 8)
  uint16_t* y;             // [H] bf16
  DecSync* sync;
};

template <class T>
__device__ inline void put(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ inline T get(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t tagged(uint32_t tag, uint32_t payload) {
  return (static_cast<uint64_t>(tag) << 32) | payload;
}

// Read words[0 .. n) into out[] (payloads) until every word carries `tag`.
__device__ inline void poll_words(const uint64_t* words, int n, uint32_t tag, uint32_t* out, uint32_t* timeout) {
  for (uint32_t it = 0;; ++it) {
    int ok = 1;
    for (int i = threadIdx.x; i < n; i += kDecThreads) {
      const uint64_t v = get(words + i);
      ok &= static_cast<uint32_t>(v >> 32) == tag;
      out[i] = static_cast<uint32_t>(v);
    }
    if (__syncthreads_and(ok)) return;
    if (it >= kSpinLimit) {
      if (threadIdx.x == 0) put(timeout, 1u);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Gate/up rows of two adjacent h columns (2p, 2p+1) of one expert: rows
// gate 2p, gate 2p+1, up 2p, up 2p+1; KCG chunks of 32 K per lane.
template <int KCG>
struct GuPair {
  uint4 c[4][KCG];
  uint16_t s[4][KCG], b[4][KCG];
};

template <int KCG>
__device__ inline void load_gu(const moe_q4& q, int64_t e, int Ih, int p, int H, int lane, GuPair<KCG>& r) {
  const int64_t base = e * 2 * static_cast<int64_t>(Ih);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t row = base + (g >> 1) * Ih + 2 * p + (g & 1);
#pragma unroll
    for (int c = 0; c < KCG; ++c) {
      const int k0 = 32 * lane + 2048 * c;
      if (k0 < H) {
        r.c[g][c] = *reinterpret_cast<const uint4*>(q.codes + row * (H / 2) + k0 / 2);
        r.s[g][c] = q.scales[row * (H / 64) + k0 / 64];
        r.b[g][c] = q.biases[row * (H / 64) + k0 / 64];
      }
    }
  }
}

// bf16(silu(gate) * up) of both columns against x (KCG x 4 uint4 per lane),
// packed (column 2p in the low half); the same in every lane.
template <int KCG>
__device__ inline uint32_t swiglu_pair(const GuPair<KCG>& r, const uint4 (&xv)[KCG][4], int H, int lane) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int c = 0; c < KCG; ++c)
      if (32 * lane + 2048 * c < H) {
        const DqConst dc = dq_const(r.s[g][c], r.b[g][c]);
        acc[g] = dot8(r.c[g][c].x, dc, xv[c][0], acc[g]);
        acc[g] = dot8(r.c[g][c].y, dc, xv[c][1], acc[g]);
        acc[g] = dot8(r.c[g][c].z, dc, xv[c][2], acc[g]);
        acc[g] = dot8(r.c[g][c].w, dc, xv[c][3], acc[g]);
      }
  float v[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) v[g] = wave_sum(acc[g]);
  const float h0 = v[0] / (1.0f + __expf(-v[0])) * v[2];
  const float h1 = v[1] / (1.0f + __expf(-v[1])) * v[3];
  return pack_bf16x2(h0, h1);
}

// One down row of one slot, KCD chunks of 8 K per lane.
template <int KCD>
struct DnRow {
  uint32_t c[KCD];
  uint16_t s[KCD], b[KCD];
};

template <int KCD>
__device__ inline void load_dn(const moe_q4& q, int64_t e, int K, int n, int H, int lane, DnRow<KCD>& r) {
  const int64_t row = e * H + n;
#pragma unroll
  for (int c = 0; c < KCD; ++c) {
    const int k0 = 8 * lane + 512 * c;
    if (k0 < K) {
      r.c[c] = *reinterpret_cast<const uint32_t*>(q.codes + row * (K / 2) + k0 / 2);
      r.s[c] = q.scales[row * (K / 64) + k0 / 64];
      r.b[c] = q.biases[row * (K / 64) + k0 / 64];
    }
  }
}

template <int KCD>
__device__ inline float dot_dn(const DnRow<KCD>& r, const uint16_t* hrow, int K, int lane) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < KCD; ++c) {
    const int k0 = 8 * lane + 512 * c;
    if (k0 < K) acc = dot8(r.c[c], dq_const(r.s[c], r.b[c]), *reinterpret_cast<const uint4*>(hrow + k0), acc);
  }
  return acc;
}

constexpr int kDecTasks = 2;    // routed gate/up (slot, column pair) tasks per wave and pass
constexpr int kDecMaxK = 16;

template <int KCG, int KCD>
__global__ __launch_bounds__(kDecThreads) void k_decode_layer(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t hs32[];  // h of all slots, [k+1][ldh/2] bf16 pairs
  __shared__ float red[2][kDecWaves];
  __shared__ int s_e[kDecMaxK];
  __shared__ float s_w[kDecMaxK + 1];                              // [k] = shared gate
  __shared__ uint32_t s_l[256 + 1];                                // logits, shared logit (fp32 bits)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int G = gridDim.x;
  const int NW = G * kDecWaves;
  const int gw = blockIdx.x * kDecWaves + wv;
  const int H = a.H, I = a.I, Is = a.Is, E = a.E, k = a.k;
  const int hp = a.ldh / 2;                   // h words per slot
  DecSync* sy = a.sync;
  const uint32_t tag = get(&sy->gen[blockIdx.x]) + 1u;
  uint64_t* lw = sy->words;                   // [E + 1]
  uint64_t* hw = lw + (E + 1);                // [k + 1][hp]

  // ---- A: loads independent of routing
  uint4 xv[KCG][4];   // x in the gate/up lane layout: K = [32 lane + 2048 c, +32)
#pragma unroll
  for (int c = 0; c < KCG; ++c)
    if (32 * lane + 2048 * c < H)
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[c][i] = *reinterpret_cast<const uint4*>(a.x + 32 * lane + 2048 * c + 8 * i);
  // router rows of this block: r = blockIdx.x + G * i (row E = shared gate weights)
  float4 rw[2][KCG];
  uint2 rx[KCG];
#pragma unroll
  for (int c = 0; c < KCG; ++c) {
    const int kk = 4 * tid + 2048 * c;
    if (kk < H) {
      rx[c] = *reinterpret_cast<const uint2*>(a.x + kk);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = blockIdx.x + G * i;
        if (r <= E)
          rw[i][c] = *reinterpret_cast<const float4*>((r < E ? a.router_w + static_cast<int64_t>(r) * H : a.wsg) + kk);
      }
    }
  }
  // shared expert column pair of this wave: p = blockIdx.x + G * wv
  const int p_sh = blockIdx.x + G * wv;
  const bool has_sh = p_sh < Is / 2;
  GuPair<KCG> sh;
  if (has_sh) load_gu<KCG>(a.sgu, 0, Is, p_sh, H, lane, sh);
  // output rows of this wave: n = gw + NW * i
  constexpr int kRowsMax = KCG;   // H <= 2048 * KCG = NW * KCG rows
  DnRow<KCD> dsh[kRowsMax];
#pragma unroll
  for (int i = 0; i < kRowsMax; ++i) {
    const int n = gw + NW * i;
    if (n < H) load_dn<KCD>(a.sdn, 0, Is, n, H, lane, dsh[i]);
  }

  // ---- B: router dot products
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < KCG; ++c) {
      const int kk = 4 * tid + 2048 * c;
      if (kk < H && blockIdx.x + G * i <= E) {
        acc = __builtin_fmaf(__uint_as_float(rx[c].x << 16), rw[i][c].x, acc);
        acc = __builtin_fmaf(__uint_as_float(rx[c].x & 0xFFFF0000u), rw[i][c].y, acc);
        acc = __builtin_fmaf(__uint_as_float(rx[c].y << 16), rw[i][c].z, acc);
        acc = __builtin_fmaf(__uint_as_float(rx[c].y & 0xFFFF0000u), rw[i][c].w, acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) red[i][wv] = acc;
  }
  __syncthreads();
  if (tid < 2) {
    const int r = blockIdx.x + G * tid;
    if (r <= E) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) l += red[tid][w];
      if (r < E && a.router_bias) l += a.router_bias[r];
      put(lw + r, tagged(tag, __float_as_uint(l)));
    }
  }

  // ---- C: shared expert column pair
  if (has_sh) {
    const uint32_t hv = swiglu_pair<KCG>(sh, xv, H, lane);
    if (lane == 0) put(hw + static_cast<int64_t>(k) * hp + p_sh, tagged(tag, hv));
  }

  // ---- D: routing decision (every block)
  poll_words(lw, E + 1, tag, s_l, &sy->timeout);
  if (wv == 0) {
    int te[16];
    float tv[16], w[16];
    topk_wave64(reinterpret_cast<const float*>(s_l), E, k, te, tv);
    topk_weights(k, tv, w);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r == lane && r < k) {
        s_e[r] = te[r];
        s_w[r] = w[r];
      }
    if (lane == 0) s_w[k] = sigmoidf_(__uint_as_float(s_l[E]));
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = tid; i < E; i += kDecThreads) a.logits[i] = __uint_as_float(s_l[i]);
    if (tid == 0) a.s_logit[0] = __uint_as_float(s_l[E]);
    if (tid < k) {
      a.ids[tid] = s_e[tid];
      a.wts[tid] = s_w[tid];
    }
    if (tid == 0) a.gate[0] = s_w[k];
  }

  // ---- E + F: routed gate/up column pairs, task q = slot * (I/2) + pair
  const int ip = I / 2;
  const int n_tasks = k * ip;
  for (int q0 = gw; q0 < n_tasks; q0 += NW * kDecTasks) {
    GuPair<KCG> ru[kDecTasks];
#pragma unroll
    for (int t = 0; t < kDecTasks; ++t) {
      const int q = q0 + NW * t;
      if (q < n_tasks) load_gu<KCG>(a.gu, s_e[q / ip], I, q % ip, H, lane, ru[t]);
    }
#pragma unroll
    for (int t = 0; t < kDecTasks; ++t) {
      const int q = q0 + NW * t;
      if (q < n_tasks) {
        const uint32_t hv = swiglu_pair<KCG>(ru[t], xv, H, lane);
        if (lane == 0) put(hw + static_cast<int64_t>(q / ip) * hp + q % ip, tagged(tag, hv));
      }
    }
  }
  // routed down rows of this wave (issued before waiting for h)
  DnRow<KCD> dr[kRowsMax][kDecMaxK];
#pragma unroll
  for (int i = 0; i < kRowsMax; ++i) {
    const int n = gw + NW * i;
#pragma unroll
    for (int j = 0; j < kDecMaxK; ++j)
      if (n < H && j < k) load_dn<KCD>(a.dn, s_e[j], I, n, H, lane, dr[i][j]);
  }

  // ---- G: all of h, then down GEMV and combine
  {
    const int nw = (k + 1) * hp;
    for (uint32_t it = 0;; ++it) {
      int ok = 1;
      for (int i = tid; i < nw; i += kDecThreads) {
        const int j = i / hp, pp = i % hp;
        if (pp < (j < k ? ip : Is / 2)) {
          const uint64_t v = get(hw + i);
          ok &= static_cast<uint32_t>(v >> 32) == tag;
          hs32[i] = static_cast<uint32_t>(v);
        }
      }
      if (__syncthreads_and(ok)) break;
      if (it >= kSpinLimit) {
        if (tid == 0) put(&sy->timeout, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  const uint16_t* hs = reinterpret_cast<const uint16_t*>(hs32);
#pragma unroll
  for (int i = 0; i < kRowsMax; ++i) {
    const int n = gw + NW * i;
    if (n < H) {
      float yv = 0.f;
#pragma unroll
      for (int j = 0; j < kDecMaxK; ++j)
        if (j < k) yv = __builtin_fmaf(s_w[j], dot_dn<KCD>(dr[i][j], hs + j * a.ldh, I, lane), yv);
      yv = __builtin_fmaf(s_w[k], dot_dn<KCD>(dsh[i], hs + k * a.ldh, Is, lane), yv);
      yv = wave_sum(yv);
      if (lane == 0) a.y[n] = f32_to_bf16_bits(yv);
    }
  }

  // ---- this block has completed the call
  if (tid == 0) put(&sy->gen[blockIdx.x], tag);
}

bool decode_supported(const moe_dims& d) {
  return d.hidden <= 2 * 2048 && d.inter <= 2 * 512 && d.shared_inter <= 2 * 512 && d.top_k <= kDecMaxK;
}

size_t decode_sync_bytes(const moe_dims& d) {
  const size_t ldh = static_cast<size_t>(div_up(max(d.inter, d.shared_inter), 8) * 8);
  return offsetof(DecSync, words) + 8 * (static_cast<size_t>(d.n_experts) + 1 + (d.top_k + 1) * ldh / 2);
}

template <int KCG, int KCD>
static void launch_dec(const DecArgs& a, size_t shbytes, hipStream_t s) {
  hipLaunchKernelGGL((k_decode_layer<KCG, KCD>), dim3(kDecBlocks), dim3(kDecThreads), shbytes, s, a);
}

hipError_t launch_decode_layer(const moe_dims& d, const moe_layer& L, const uint16_t* x, uint16_t* y,
                               const DecodePtrs& p, hipStream_t s) {
  DecArgs a{};
  a.gu = L.gate_up;
  a.dn = L.down;
  a.sgu = L.sh_gate_up;
  a.sdn = L.sh_down;
  a.router_w = L.router_w;
  a.router_bias = L.router_bias;
  a.wsg = L.shared_gate_w;
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
  a.ldh = static_cast<int>(div_up(max(d.inter, d.shared_inter), 8) * 8);
  a.y = y;
  a.sync = reinterpret_cast<DecSync*>(p.sync);
  const int kcg = static_cast<int>(div_up(d.hidden, 2048));
  const int kcd = static_cast<int>(div_up(max(d.inter, d.shared_inter), 512));
  const size_t sh = static_cast<size_t>(d.top_k + 1) * a.ldh * 2;   // h of all slots in LDS
  switch (kcg * 10 + kcd) {   // decode_supported(): both 1 or 2
    case 11: launch_dec<1, 1>(a, sh, s); break;
    case 12: launch_dec<1, 2>(a, sh, s); break;
    case 21: launch_dec<2, 1>(a, sh, s); break;
    default: launch_dec<2, 2>(a, sh, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
