// Decode path of the MoE layer: one token per step, or a few (up to kDecMaxT,
// the shapes of speculative verification).  Each touched expert's weights are
// then used once per token, so the work is matrix-vector, limited by memory
// bandwidth, and the pages assign it to the vector ALUs rather than the
// matrix units (Lily page, section "Why Apple Silicon isn't just a smaller
// datacenter GPU"); chains of kernels are fused so that intermediates stay on
// chip (Inside Lily page, section "Performance Gains and Workload Patterns").
//
// The whole layer is one launch of kDecBlocks workgroups of 8 waves, all
// resident at once:
//   A. issue the loads that need no routing decision: this block's router
//      row(s), the shared expert's gate/up rows of this wave's column pair and
//      its down rows for this wave's output row;
//   B. router dot products (fp32 weights) of every token -> logit words
//   D. every block polls the logit words until all carry this call's tag and
//      recomputes every token's top-k itself (all waves, lower expert index
//      on ties), so the routing decision needs no second round trip;
//   E. issue the routed experts' gate/up rows of this wave's (token, slot,
//      column pair) task and the down rows of every token's experts for this
//      wave's output row;
//   C. while those rows are in flight: shared expert SwiGLU column pair,
//      every token                                      -> h words of slot k
//   F. routed SwiGLU column pairs                       -> h words of slot j
//   G. poll the h words; down GEMV over each token's k+1 slots with the
//      weighted combine in registers, slot order, shared expert last -> y.
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
// a CU; the host checks the device's residency before it launches), so every
// wait ends; a wait that exceeds kSpinLimit polls sets the hand-over timeout
// bit of the workspace's error word and carries on, so a launch always
// completes.
#include "gemv.hpp"
#include "topk.hpp"

namespace moe {

constexpr int kDecBlocks = 256;
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr uint32_t kSpinLimit = 1u << 22;

// Workspace words of the fused path (zero before the first call).
struct DecSync {
  uint32_t gen[kDecBlocks];   // calls completed, per block
  uint32_t pad[64];
  uint64_t words[1];          // logit words [T][E + 1], then h words [T][k + 1][ldh / 2]
};

struct DecArgs {
  moe_q4 gu, dn, sgu, sdn;
  const float* router_w;   // [E][H]
  const float* router_bias;
  const float* wsg;        // [H]
  int H, I, Is, E, k, T;
  const uint16_t* x;       // [T][H] bf16
  float* logits;           // [T][E]
  float* s_logit;          // [T]
  int32_t* ids;            // [T][k]
  float* wts;              // [T][k]
  float* gate;             // [T]
  int ldh;                 // h row stride (multiple of 8)
  uint16_t* y;             // [T][H] bf16
  DecSync* sync;
  uint32_t* err;           // the workspace's device error word
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

// Read the words i < n with live(i) into out[i] (payloads) until every one has
// carried `tag`.  Thread t owns words t + kDecThreads * m, m < M: it requests
// its pending words together, up to C at a time (so at most C owned words cost
// one memory round trip per round), and a word once seen with the tag is not
// requested again.  The block agrees on "all done" with one barrier per round:
// wave w writes its verdict to done[round & 1][w] (a wave cannot reach round
// r + 2's write before every wave has passed round r + 1's barrier, that is,
// has read round r's verdicts).
template <int M, int C, class Live>
__device__ inline void poll_words(const uint64_t* words, int n, uint32_t tag, uint32_t* out, uint32_t* err,
                                  Live live, uint32_t (&done)[2][kDecWaves]) {
  const int tid = threadIdx.x;
  uint32_t pending = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int i = tid + kDecThreads * m;
    if (i < n && live(i)) pending |= 1u << m;
  }
  for (uint32_t it = 0;; ++it) {
#pragma unroll
    for (int m0 = 0; m0 < M; m0 += C) {
      uint64_t v[C];
#pragma unroll
      for (int m = m0; m < m0 + C && m < M; ++m)
        if (pending >> m & 1u) v[m - m0] = get(words + tid + kDecThreads * m);
#pragma unroll
      for (int m = m0; m < m0 + C && m < M; ++m)
        if ((pending >> m & 1u) && static_cast<uint32_t>(v[m - m0] >> 32) == tag) {
          out[tid + kDecThreads * m] = static_cast<uint32_t>(v[m - m0]);
          pending &= ~(1u << m);
        }
    }
    const bool wave_done = __ballot(pending != 0u) == 0;
    if ((tid & 63) == 0) done[it & 1u][tid >> 6] = wave_done ? 1u : 0u;
    __syncthreads();
    uint32_t all = 1u;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) all &= done[it & 1u][w];
    if (all) return;
    if (it >= kSpinLimit) {
      if (tid == 0)
        __hip_atomic_fetch_or(err, static_cast<uint32_t>(MOE_DEVERR_HANDOVER_TIMEOUT), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// routed gate/up (slot, column pair) tasks per wave and pass: two rows' loads in
// flight where they fit the registers (hidden <= 2048), else one
template <int KCG>
constexpr int kDecTasks = KCG == 1 ? 2 : 1;
constexpr int kDecMaxK = 16;
constexpr int kDecMaxE = 256;
static_assert(kDecMaxE + 1 <= kDecThreads, "one token's logit words: at most one per thread");
static_assert(kDecMaxE == 32 * kDecWaves, "top-k stage 1 gives each wave 32 experts");
static_assert(kDecMaxT <= kDecWaves, "several tokens: one wave per token's top-k");

// Top-k (k <= 16) of the E <= 256 logits (fp32 bits in l[]) by the whole
// block, in the order larger logit first, then lower expert index (-0 and +0
// tie).  Expert i's place in that order is fixed by a unique 64-bit key: the
// order-preserving 32-bit image of its logit, then 255 - i (experts i >= E
// get the key 255 - i, below every real one), so its rank is the number of
// larger keys.
//   1. wave w ranks experts 32w .. 32w + 31 among themselves, each half-wave
//      counting against 16 of them; an expert outranked by k others of its
//      own wave cannot be in the first k, so each wave passes on its first k;
//   2. a survivor's overall rank is the number of larger survivors: wave w
//      counts, for every survivor, the larger ones among wave w's k (for its
//      own wave that count is its local rank), and the eight counts are
//      summed; the survivor of rank r < k writes slot r (expert, logit).
// Every thread of the block must call it; it ends with a barrier.
__device__ inline void topk_block(const uint32_t* l, int E, int k, uint64_t* key, uint64_t* cand,
                                  int (*part)[kDecWaves * kDecMaxK], int* top_e, float* top_v) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid < kDecMaxE)
    key[tid] = tid < E ? (static_cast<uint64_t>(topk_key32(__uint_as_float(l[tid]))) << 8) | (255u - tid)
                       : static_cast<uint64_t>(255u - tid);
  __syncthreads();
  {
    const uint64_t ki = key[32 * wv + (lane & 31)];
    const uint64_t* kj = key + 32 * wv + 16 * (lane >> 5);
    int r = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) r += kj[j] > ki ? 1 : 0;
    r += __shfl_xor(r, 32);
    if (lane < 32 && r < k) cand[wv * k + r] = ki;
  }
  __syncthreads();
  const int nc = kDecWaves * k;
  const uint64_t* mine = cand + wv * k;
#pragma unroll
  for (int c0 = 0; c0 < kDecWaves * kDecMaxK; c0 += 64) {
    const int c = c0 + lane;
    if (c0 < nc) {
      int cnt = 0;
      if (c < nc) {
        const uint64_t kc = cand[c];
#pragma unroll
        for (int r = 0; r < kDecMaxK; ++r)
          if (r < k) cnt += mine[r] > kc ? 1 : 0;
      }
      part[wv][c] = cnt;
    }
  }
  __syncthreads();
  if (tid < nc) {
    int g = 0;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) g += part[w][tid];
    if (g < k) {
      const uint64_t kc = cand[tid];
      top_e[g] = 255 - static_cast<int>(kc & 255u);
      top_v[g] = topk_key32_value(static_cast<uint32_t>(kc >> 8));
    }
  }
  __syncthreads();
}

// KMAX: bound on k the registers are sized for (8 or 16); TM: bound on the
// number of tokens (1, or kDecMaxT for the multi-token form).
template <int KCG, int KCD, int KMAX, int TM>
__global__ __launch_bounds__(kDecThreads) void k_decode_layer(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t hs32[];  // h of all slots, [T][k+1][ldh/2] bf16 pairs
  __shared__ float red[2][TM][kDecWaves];
  __shared__ int s_e[TM][kDecMaxK];
  __shared__ float s_v[TM][kDecMaxK];                              // top-k logits
  __shared__ float s_w[kDecWaves][TM][kDecMaxK + 1];               // weights, [k] = shared gate; per wave
  __shared__ uint32_t s_l[TM][kDecMaxE + 1];                       // logits, shared logit (fp32 bits)
  __shared__ uint64_t s_key[kDecMaxE];
  __shared__ uint64_t s_cand[kDecWaves * kDecMaxK];
  __shared__ int s_part[kDecWaves][kDecWaves * kDecMaxK];
  __shared__ uint32_t s_done[2][kDecWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int G = gridDim.x;
  const int NW = G * kDecWaves;
  const int gw = blockIdx.x * kDecWaves + wv;
  const int H = a.H, I = a.I, Is = a.Is, E = a.E, k = a.k;
  const int T = TM == 1 ? 1 : a.T;
  const int hp = a.ldh / 2;                   // h words per slot
  DecSync* sy = a.sync;
  const uint32_t tag = get(&sy->gen[blockIdx.x]) + 1u;
  uint64_t* lw = sy->words;                   // [T][E + 1]
  uint64_t* hw = lw + T * (E + 1);            // [T][k + 1][hp]

  // ---- A: loads independent of routing
  uint4 xv[TM][KCG][4];   // x in the gate/up lane layout: K = [32 lane + 2048 c, +32)
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int c = 0; c < KCG; ++c)
      if (t < T && 32 * lane + 2048 * c < H)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xv[t][c][i] = *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(t) * H + 32 * lane + 2048 * c + 8 * i);
  // router rows of this block: r = blockIdx.x + G * i (row E = shared gate weights)
  float4 rw[2][KCG];
  uint2 rx[TM][KCG];
#pragma unroll
  for (int c = 0; c < KCG; ++c) {
    const int kk = 4 * tid + 2048 * c;
    if (kk < H) {
#pragma unroll
      for (int t = 0; t < TM; ++t)
        if (t < T) rx[t][c] = *reinterpret_cast<const uint2*>(a.x + static_cast<int64_t>(t) * H + kk);
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

  // ---- B: router dot products, every token against this block's rows
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t >= T) continue;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < KCG; ++c) {
        const int kk = 4 * tid + 2048 * c;
        if (kk < H && blockIdx.x + G * i <= E) {
          acc = __builtin_fmaf(__uint_as_float(rx[t][c].x << 16), rw[i][c].x, acc);
          acc = __builtin_fmaf(__uint_as_float(rx[t][c].x & 0xFFFF0000u), rw[i][c].y, acc);
          acc = __builtin_fmaf(__uint_as_float(rx[t][c].y << 16), rw[i][c].z, acc);
          acc = __builtin_fmaf(__uint_as_float(rx[t][c].y & 0xFFFF0000u), rw[i][c].w, acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) red[i][t][wv] = acc;
    }
  __syncthreads();
  if (tid < 2 * T) {
    const int i = tid / T, t = tid - i * T;
    const int r = blockIdx.x + G * i;
    if (r <= E) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) l += red[i][t][w];
      if (r < E && a.router_bias) l += a.router_bias[r];
      put(lw + t * (E + 1) + r, tagged(tag, __float_as_uint(l)));
    }
  }

  // ---- C: shared expert column pair, every token.  In the one-token form
  // with hidden <= 2048 it runs after the routing decision, while the routed
  // rows are in flight (it needs no routing, and before the logit poll it
  // would only delay the routing decision); the wider and multi-token forms
  // have no registers to hold its rows that long, and run it here.
  constexpr bool kLateShared = TM == 1 && KCG == 1;
  if constexpr (!kLateShared) {
    if (has_sh) {
#pragma unroll
      for (int t = 0; t < TM; ++t)
        if (t < T) {
          const uint32_t hv = swiglu_pair<KCG>(sh, xv[t], H, lane);
          if (lane == 0) put(hw + (static_cast<int64_t>(t) * (k + 1) + k) * hp + p_sh, tagged(tag, hv));
        }
    }
  }

  // ---- D: routing decision of every token (every block)
  poll_words<(TM * (kDecMaxE + 1) + kDecThreads - 1) / kDecThreads, (TM * (kDecMaxE + 1) + kDecThreads - 1) / kDecThreads>(
      lw, T * (E + 1), tag, &s_l[0][0], a.err, [](int) { return true; }, s_done);
  if constexpr (TM > 1) {
    // the polled words are [T][E + 1]; the rows of s_l are kDecMaxE + 1 apart
    for (int t = T - 1; t > 0; --t) {
      uint32_t v = 0;
      if (tid <= E) v = (&s_l[0][0])[t * (E + 1) + tid];
      __syncthreads();
      if (tid <= E) s_l[t][tid] = v;
      __syncthreads();
    }
  }
  // renormalised weights exp(l_r - l_0) / sum_r' exp(l_r' - l_0), the sum in
  // slot order: lane t k + r takes token t's slot r exponential.  Every wave
  // computes them (the same values) into its own rows of s_w, so no further
  // barrier is needed; [k] = shared gate
  if constexpr (TM == 1) {
    topk_block(s_l[0], E, k, s_key, s_cand, s_part, s_e[0], s_v[0]);
  } else {
    // several tokens: wave t takes token t's top-k on its own (eight rounds of
    // a wave-wide maximum, the same order), all tokens at once
    if (wv < T) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = lane + 64 * i < E ? __uint_as_float(s_l[wv][lane + 64 * i]) : 0.f;
      if (k == 8) {
        int my_e;
        float my_v;
        topk_wave64_fixed<8>(v, E, my_e, my_v);
        if (lane < 8) {
          s_e[wv][lane] = my_e;
          s_v[wv][lane] = my_v;
        }
      } else {
        int te[16];
        float tv[16];
        topk_wave64_regs(v, E, k, te, tv);
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (lane == r && r < k) {
            s_e[wv][r] = te[r];
            s_v[wv][r] = tv[r];
          }
      }
    }
    __syncthreads();
  }
  {
    const int tl = min(lane / k, TM - 1), rl = lane - tl * k;   // (lanes past T k hold nothing)
    const bool mine = lane < T * k;
    const float ex = mine ? expf(s_v[tl][rl] - s_v[tl][0]) : 0.f;
    float inv = 0.f;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t >= T) continue;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < kDecMaxK; ++r)
        if (r < k) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), t * k + r));
      const float it = 1.0f / sum;
      if (tl == t) inv = it;
    }
    if (mine) s_w[wv][tl][rl] = ex * inv;
    if (lane < T) s_w[wv][lane][k] = sigmoidf_(__uint_as_float(s_l[lane][E]));
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's s_w rows are written
  __builtin_amdgcn_wave_barrier();
  if (blockIdx.x == 0) {
    for (int t = 0; t < T; ++t) {
      for (int i = tid; i < E; i += kDecThreads) a.logits[t * E + i] = __uint_as_float(s_l[t][i]);
      if (tid == 0) a.s_logit[t] = __uint_as_float(s_l[t][E]);
      if (tid < k) {
        a.ids[t * k + tid] = s_e[t][tid];
        a.wts[t * k + tid] = s_w[0][t][tid];
      }
      if (tid == 0) a.gate[t] = s_w[0][t][k];
    }
  }

  // ---- E + F: routed gate/up column pairs, task q = (token * k + slot) * (I/2)
  // + pair.  With hidden <= 2048 this wave's routed down rows are requested
  // right after its first gate/up rows, so they arrive while h is being
  // produced and handed over (wider rows leave no registers for that: there
  // they follow the gate/up work).
  const int ip = I / 2;
  const int n_tasks = T * k * ip;
  DnRow<KCD> dr[kRowsMax][TM * KMAX];
  auto load_down = [&]() {
#pragma unroll
    for (int i = 0; i < kRowsMax; ++i) {
      const int n = gw + NW * i;
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (n < H && t < T && j < k) load_dn<KCD>(a.dn, s_e[t][j], I, n, H, lane, dr[i][t * KMAX + j]);
    }
  };
  // Every wave runs the first round, even without a task: there, right after
  // requesting its first gate/up rows, it requests its routed down rows (with
  // hidden <= 2048) and computes the late shared pair while the rows are in
  // flight.
  bool first = true;
  for (int q0 = gw;; q0 += NW * kDecTasks<KCG>) {
    GuPair<KCG> ru[kDecTasks<KCG>];
    uint4 xq[TM == 1 ? 1 : kDecTasks<KCG>][KCG][4];   // the task's token (one token: xv)
#pragma unroll
    for (int u = 0; u < kDecTasks<KCG>; ++u) {
      const int q = q0 + NW * u;
      if (q < n_tasks) {
        const int slot = q / ip, t = slot / k;
        load_gu<KCG>(a.gu, s_e[t][slot - t * k], I, q % ip, H, lane, ru[u]);
        if constexpr (TM > 1) {
#pragma unroll
          for (int c = 0; c < KCG; ++c)
            if (32 * lane + 2048 * c < H)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                xq[u][c][i] =
                    *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(t) * H + 32 * lane + 2048 * c + 8 * i);
        }
      }
    }
    if (first) {
      if constexpr (KCG == 1) load_down();
      if constexpr (kLateShared) {
        if (has_sh) {   // one token (TM == 1)
          const uint32_t hv = swiglu_pair<KCG>(sh, xv[0], H, lane);
          if (lane == 0) put(hw + static_cast<int64_t>(k) * hp + p_sh, tagged(tag, hv));
        }
      }
      first = false;
    }
#pragma unroll
    for (int u = 0; u < kDecTasks<KCG>; ++u) {
      const int q = q0 + NW * u;
      if (q < n_tasks) {
        const int slot = q / ip, t = slot / k;
        uint32_t hv;
        if constexpr (TM == 1)
          hv = swiglu_pair<KCG>(ru[u], xv[0], H, lane);
        else
          hv = swiglu_pair<KCG>(ru[u], xq[u], H, lane);
        if (lane == 0) put(hw + (static_cast<int64_t>(slot) + t) * hp + q % ip, tagged(tag, hv));
      }
    }
    if (q0 + NW * kDecTasks<KCG> >= n_tasks) break;
  }
  if constexpr (KCG != 1) load_down();

  // ---- G: all of h, then down GEMV and combine, every token
  constexpr int kHWords = TM * (KMAX + 1) * 256 * KCD;   // T (k + 1) slots of at most 512 KCD columns
  constexpr int kHPerThread = (kHWords + kDecThreads - 1) / kDecThreads;
  // (the widest form, k > 8 with hidden and inter both past 2048 / 512, has no
  // registers to spare: there one word is requested at a time)
  constexpr int kHChunk = KCG * KCD == 4 && KMAX > 8 ? 1 : (kHPerThread < 9 ? kHPerThread : 9);
  poll_words<kHPerThread, kHChunk>(
      hw, T * (k + 1) * hp, tag, hs32, a.err,
      [&](int i) {
        const int slot = i / hp;
        const int j = slot % (k + 1);
        return i - slot * hp < (j < k ? ip : Is / 2);
      },
      s_done);
  const uint16_t* hs = reinterpret_cast<const uint16_t*>(hs32);
#pragma unroll
  for (int i = 0; i < kRowsMax; ++i) {
    const int n = gw + NW * i;
    if (n < H) {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t >= T) continue;
        const float* sw = s_w[wv][t];
        const uint16_t* ht = hs + static_cast<int64_t>(t) * (k + 1) * a.ldh;
        float yv = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k) yv = __builtin_fmaf(sw[j], dot_dn<KCD>(dr[i][t * KMAX + j], ht + j * a.ldh, I, lane), yv);
        yv = __builtin_fmaf(sw[k], dot_dn<KCD>(dsh[i], ht + k * a.ldh, Is, lane), yv);
        yv = wave_sum(yv);
        if (lane == 0) a.y[static_cast<int64_t>(t) * H + n] = f32_to_bf16_bits(yv);
      }
    }
  }

  // ---- this block has completed the call
  if (tid == 0) put(&sy->gen[blockIdx.x], tag);
}

bool decode_supported(const moe_dims& d, int T) {
  if (T == 1)
    return d.hidden <= 2 * 2048 && d.inter <= 2 * 512 && d.shared_inter <= 2 * 512 && d.top_k <= kDecMaxK;
  return T >= 2 && T <= kDecMaxT && d.hidden <= 2048 && d.inter <= 512 && d.shared_inter <= 512 && d.top_k <= 8;
}

size_t decode_sync_bytes(const moe_dims& d) {
  const size_t ldh = static_cast<size_t>(div_up(max(d.inter, d.shared_inter), 8) * 8);
  const size_t T = kDecMaxT;
  return offsetof(DecSync, words) + 8 * T * (static_cast<size_t>(d.n_experts) + 1 + (d.top_k + 1) * ldh / 2);
}

template <int KCG, int KCD>
static const void* dec_kernel(int k) {
  return k <= 8 ? reinterpret_cast<const void*>(&k_decode_layer<KCG, KCD, 8, 1>)
                : reinterpret_cast<const void*>(&k_decode_layer<KCG, KCD, kDecMaxK, 1>);
}

// The kernel instantiation and dynamic LDS bytes of the fused layer for (d, T),
// where decode_supported(d, T).
static const void* dec_plan(const moe_dims& d, int T, size_t* shbytes) {
  const size_t ldh = static_cast<size_t>(div_up(max(d.inter, d.shared_inter), 8) * 8);
  *shbytes = static_cast<size_t>(T) * (d.top_k + 1) * ldh * 2;   // h of all slots in LDS
  if (T > 1)   // decode_supported(): hidden <= 2048, inter and shared_inter <= 512, k <= 8
    return reinterpret_cast<const void*>(&k_decode_layer<1, 1, 8, kDecMaxT>);
  const int kcg = static_cast<int>(div_up(d.hidden, 2048));
  const int kcd = static_cast<int>(div_up(max(d.inter, d.shared_inter), 512));
  switch (kcg * 10 + kcd) {   // decode_supported(): both 1 or 2
    case 11: return dec_kernel<1, 1>(d.top_k);
    case 12: return dec_kernel<1, 2>(d.top_k);
    case 21: return dec_kernel<2, 1>(d.top_k);
    default: return dec_kernel<2, 2>(d.top_k);
  }
}

hipError_t decode_residency(const moe_dims& d, int T, int* needed, int* resident) {
  *needed = kDecBlocks;
  *resident = 0;
  size_t sh = 0;
  const void* kern = dec_plan(d, T, &sh);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kDecThreads, sh);
  if (e != hipSuccess) return e;
  *resident = cus * per_cu;
  return hipSuccess;
}

hipError_t launch_decode_layer(const moe_dims& d, const moe_layer& L, const uint16_t* x, int T, uint16_t* y,
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
  a.T = T;
  a.x = x;
  a.logits = p.logits;
  a.s_logit = p.s_logit;
  a.ids = p.ids;
  a.wts = p.wts;
  a.gate = p.gate;
  a.ldh = static_cast<int>(div_up(max(d.inter, d.shared_inter), 8) * 8);
  a.y = y;
  a.sync = reinterpret_cast<DecSync*>(p.sync);
  a.err = p.err;
  size_t sh = 0;
  const void* kern = dec_plan(d, T, &sh);
  void* args[] = {&a};
  return hipLaunchKernel(kern, dim3(kDecBlocks), dim3(kDecThreads), args, sh, s);
}

}  // namespace moe
