// attn.hip -- one decode step of grouped-query attention.
//
// The model whose MoE layer this library runs interleaves its MoE layers with
// full-attention layers in which 16 query heads share 2 key/value heads
// ("Lily: Perplexity's Custom Inference Engine for Apple Silicon", section "The
// architecture that forces the issue").  At decode the step reads the whole
// key/value cache for one query row per head.  The "Inside Lily ..." page lists
// GQA packing among its optimisations (section "Key Optimizations at a
// Glance"): the query heads of a group share one load of each key/value row
// instead of loading it once per query head.
//
// Here one workgroup owns (sequence, key/value head, range of positions) and
// all the group's query heads (at most 8).  Its eight waves work independently:
// wave w takes the 16-position stages w, w + 8, ... of the range.  A wave
// brings a stage's 16 key and 16 value rows into its own LDS slots with
// direct-to-LDS loads (16-byte chunks XOR-swizzled by row, so that the
// fragment reads below are conflict-free), the next stage's keys being
// requested as soon as the current scores are formed and its values as soon
// as the current values are used; no workgroup barrier is needed until the
// end.  Scores are one v_mfma_f32_16x16x32_bf16 chain per stage (16 positions
// x 16 query-head columns, the key rows as the first operand and the query
// rows, held in registers, as the second; columns past the group are zero).
// An online softmax keeps each head's running maximum and sum.  The weighted
// value sum is a second MFMA chain, v_mfma_f32_16x16x16_bf16 per 16 value
// columns, computing the transposed output (value columns x heads): the score
// registers already hold the probabilities in the layout of its second
// operand, split exactly into a bf16 high part and a bf16 remainder (two
// MFMAs, so they keep 16 significant bits), and the first operand is the
// value rows read column-wise from LDS.  At the end the waves' states
// are combined in wave order, and each range leaves its (maximum, sum,
// unnormalised output) in the workspace; k_gqa_merge combines a head's ranges
// in range order, so the result does not depend on scheduling.  With one
// query head per workgroup (pack_heads == 0) the same kernel reads each
// key/value row once per query head: the unpacked form the packing is
// measured against.

#include "internal.hpp"
#include "attn.hpp"

namespace moe {

namespace {

constexpr int kAtPos = 16;        // positions per stage: the rows of one 16x16x32 MFMA
constexpr int kAtWaves = 8;
constexpr int kAtThreads = 64 * kAtWaves;
constexpr int kMgThreads = 256;   // merge
constexpr int kAtGroup = 8;       // query heads per workgroup at most
constexpr int kAtTarget = 2048 / kAtWaves;   // workgroups wanted per launch: eight waves per CU (16 KB of LDS each)

template <int D>
struct AtGeom {
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kSlot = kAtPos * kRowBytes;    // the key (or value) rows of one stage
  static constexpr int kLoads = kSlot / 1024;         // 1 KB direct loads per slot and wave
  // XOR key of row r: rows sharing a 256-byte bank line get distinct keys
  static constexpr int kShift = kChunks >= 16 ? 0 : 1;
  static constexpr int kMask = (kChunks >= 16 ? 16 : kChunks) - 1;
  static_assert(kSlot % 1024 == 0, "whole 1 KB loads");
};
// Physical 16-byte chunk of logical chunk c in row r of a slot (and back: the
// XOR is its own inverse).  The 16 rows of an MFMA fragment read, and the
// chunks of one row read by the value lanes, fall in distinct bank groups.
template <int D>
__device__ inline int at_chunk(int r, int c) {
  return c ^ ((r >> AtGeom<D>::kShift) & AtGeom<D>::kMask);
}

template <int D>
struct AttnLds {
  unsigned char kv[kAtWaves][2][AtGeom<D>::kSlot];   // per wave: key slot, value slot
  float fac[kAtGroup][kAtWaves];                     // end: each wave's factor e^(m_w - M) per head
};
typedef short bf16x4 __attribute__((ext_vector_type(4)));
__device__ inline f32x4 mfma16k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ inline float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS reads have returned before a
// direct load may overwrite what they read.
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <int D>
__global__ __launch_bounds__(kAtThreads, 8 / kAtWaves) void k_gqa_partial(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kc,
                                                               const uint16_t* __restrict__ vc,
                                                               const int32_t* __restrict__ lens, int Hq, int Hkv,
                                                               int S, int gw, int rows_per_split, int n_splits,
                                                               float scale, float* __restrict__ part_o,
                                                               float* __restrict__ part_ml) {
  using G = AtGeom<D>;
  __shared__ __attribute__((aligned(1024))) AttnLds<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, b = blockIdx.z;
  const int h0 = blockIdx.y * gw;                 // first query head of this workgroup
  const int kv = h0 / (Hq / Hkv);
  const int L = min(max(lens[b], 0), S);
  const int start = split * rows_per_split;
  if (start >= L) return;                         // the merge reads only ranges below L
  const int end = min(start + rows_per_split, L);
  const int n_st = (end - start + kAtPos - 1) / kAtPos;
  const int my_st = n_st > wave ? (n_st - wave + kAtWaves - 1) / kAtWaves : 0;   // stages wave, wave + kAtWaves, ...

  // score roles: lane = (position row lane % 16 of the key fragment, query
  // head column lane % 16 of the query fragment and of the scores), lane
  // group qg = lane / 16 covering K offsets 8 qg .. 8 qg + 7 of each k-step
  const int col = lane & 15, qg = lane >> 4;
  uint4 qf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    qf[s] = uint4{0u, 0u, 0u, 0u};
    if (col < gw) {
      const uint32_t* src =
          reinterpret_cast<const uint32_t*>(q + (static_cast<int64_t>(b) * Hq + h0 + col) * D + 32 * s + 8 * qg);
      qf[s] = uint4{src[0], src[1], src[2], src[3]};
    }
  }
  // output: o[t][u] holds value column 16 t + 4 qg + u of head col (the
  // transposed product's accumulator layout)
  constexpr int kTiles = D / 16;
  f32x4 o[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;   // head col, the same in the four lane groups

  const int64_t row0 = (static_cast<int64_t>(b) * Hkv + kv) * S;   // cache row of position 0
  const i32x4 krs = buffer_rsrc(kc + row0 * D), vrs = buffer_rsrc(vc + row0 * D);
  const uint32_t kslot = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr(&sm.kv[wave][0][0]))));
  const uint32_t vslot = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr(&sm.kv[wave][1][0]))));
  // byte offsets (from the head's position 0) of this lane's 16-byte pieces of
  // a stage at p0; rows past the range re-read its last row
  uint32_t off[G::kLoads];
  auto offsets = [&](int p0) {
#pragma unroll
    for (int j = 0; j < G::kLoads; ++j) {
      const int byte = j * 1024 + lane * 16;
      const int r = byte / G::kRowBytes, ph = (byte % G::kRowBytes) / 16;
      const int p = min(p0 + r, end - 1);
      off[j] = static_cast<uint32_t>((p * D + at_chunk<D>(r, ph) * 8) * 2);
    }
  };
  auto issue = [&](const i32x4& rs, uint32_t slot) {
#pragma unroll
    for (int j = 0; j < G::kLoads; ++j) bdma16(rs, off[j], 0u, slot + j * 1024);
  };
  const unsigned char* ks = &sm.kv[wave][0][0];
  const unsigned char* vs = &sm.kv[wave][1][0];

  if (my_st > 0) {
    offsets(start + wave * kAtPos);
    issue(krs, kslot);
    issue(vrs, vslot);
  }
  for (int i = 0; i < my_st; ++i) {
    const int p0 = start + (wave + i * kAtWaves) * kAtPos;
    const int nv = min(kAtPos, end - p0);
    const bool more = i + 1 < my_st;
    wait_vmcnt<G::kLoads>();   // this stage's keys (its values may still be in flight)
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const bf16x8 kf =
          *reinterpret_cast<const bf16x8*>(ks + col * G::kRowBytes + at_chunk<D>(col, 4 * s + qg) * 16);
      sc = mfma16(kf, __builtin_bit_cast(bf16x8, qf[s]), sc);
    }
    // sc[u]: position 4 qg + u of the stage, head col
    wait_lgkm0();
    if (more) {
      offsets(p0 + kAtWaves * kAtPos);
      issue(krs, kslot);
    }
    float sv[4], mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sv[u] = 4 * qg + u < nv ? sc[u] * scale : -INFINITY;
      mx = fmaxf(mx, sv[u]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m_run, mx);   // finite: the stage's first position is live
    const float al = expf(m_run - mn);
    float ev[4], es = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ev[u] = 4 * qg + u < nv ? expf(sv[u] - mn) : 0.f;
      es += ev[u];
    }
    es += __shfl_xor(es, 16);
    es += __shfl_xor(es, 32);
    l_run = l_run * al + es;
    m_run = mn;
    // probabilities as the second operand (positions 4 qg .. 4 qg + 3 of head
    // col): high bf16 part and the bf16 remainder (both exact splits of the
    // fp32 value up to the remainder's own rounding)
    bf16x4 phi, plo;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t h = f32_to_bf16_bits(ev[u]);
      const float hv = __uint_as_float(static_cast<uint32_t>(h) << 16);
      phi[u] = static_cast<short>(h);
      plo[u] = static_cast<short>(f32_to_bf16_bits(ev[u] - hv));
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) o[t] *= al;
    if (more)
      wait_vmcnt<G::kLoads>();   // this stage's values (the next keys may still be in flight)
    else
      wait_vmcnt<0>();
    // first operand: value column 16 t + col at positions 4 qg .. 4 qg + 3
    const int vc8 = col >> 3, ve = (col & 7) * 2;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      bf16x4 va;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * qg + u;
        va[u] = *reinterpret_cast<const short*>(vs + r * G::kRowBytes + at_chunk<D>(r, 2 * t + vc8) * 16 + ve);
      }
      o[t] = mfma16k16(va, phi, o[t]);
      o[t] = mfma16k16(va, plo, o[t]);
    }
    wait_lgkm0();
    if (more) issue(vrs, vslot);
  }

  // the waves' states, combined in wave order through their own slots
  __syncthreads();
  float* mine = reinterpret_cast<float*>(&sm.kv[wave][0][0]);   // m [8], l [8], o [8][D]
  static_assert((2 * kAtGroup + kAtGroup * D) * sizeof(float) <= 2 * AtGeom<D>::kSlot, "state area");
  if (qg == 0 && col < kAtGroup) {
    mine[col] = m_run;
    mine[kAtGroup + col] = l_run;
  }
  if (col < kAtGroup) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
      *reinterpret_cast<f32x4*>(mine + 2 * kAtGroup + col * D + 16 * t + 4 * qg) = o[t];
  }
  __syncthreads();
  // per head: the range's maximum M, each wave's factor e^(m_w - M) (0 for a
  // wave with no stage, m = -inf) and the range's sum
  float* fac = &sm.fac[0][0];
  if (tid < kAtGroup) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAtWaves; ++w) M = fmaxf(M, reinterpret_cast<const float*>(&sm.kv[w][0][0])[tid]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < kAtWaves; ++w) {
      const float* st = reinterpret_cast<const float*>(&sm.kv[w][0][0]);
      const float f = expf(st[tid] - M);
      fac[tid * kAtWaves + w] = f;
      den = fmaf(f, st[kAtGroup + tid], den);
    }
    if (tid < gw) {
      float* ml = part_ml + ((static_cast<int64_t>(b) * Hq + h0 + tid) * n_splits + split) * 2;
      ml[0] = M;
      ml[1] = den;
    }
  }
  __syncthreads();
  for (int i = tid; i < gw * D; i += kAtThreads) {
    const int g = i / D, d = i % D;
    float num = 0.f;
#pragma unroll
    for (int w = 0; w < kAtWaves; ++w)
      num = fmaf(fac[g * kAtWaves + w], reinterpret_cast<const float*>(&sm.kv[w][0][0])[2 * kAtGroup + g * D + d],
                 num);
    part_o[((static_cast<int64_t>(b) * Hq + h0 + g) * n_splits + split) * D + d] = num;
  }
}

// One workgroup per (16 output columns, query head, sequence): the ranges'
// partial results combined as out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// Each of 16 split lanes per column adds ranges s = lane, lane + 16, ... in
// order, and the 16 lane sums are added in lane order, so the result does not
// depend on scheduling.
constexpr int kMergeCols = 16;
__global__ __launch_bounds__(kMgThreads) void k_gqa_merge(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int32_t* __restrict__ lens, int Hq, int S, int D,
                                                          int rows_per_split, int n_splits, uint16_t* __restrict__ out) {
  constexpr int kW = kMgThreads / 64;
  __shared__ float red[2][kW];
  __shared__ float part[kMgThreads / kMergeCols][kMergeCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * kMergeCols, h = blockIdx.y, b = blockIdx.z;
  const int L = min(max(lens[b], 0), S);
  const int ns = (L + rows_per_split - 1) / rows_per_split;
  const int64_t bh = static_cast<int64_t>(b) * Hq + h;
  if (ns == 0) {
    if (tid < kMergeCols) out[bh * D + c0 + tid] = 0;
    return;
  }
  const float* ml = part_ml + bh * n_splits * 2;
  const int c = tid % kMergeCols, sl = tid / kMergeCols;
  constexpr int kLanes = kMgThreads / kMergeCols;   // split lanes per column
  const float* po = part_o + bh * n_splits * D + c0 + c;
  // this lane's first kPre ranges, requested before the maximum is known
  constexpr int kPre = 16;
  float ov[kPre], mv[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int s = sl + i * kLanes;
    ov[i] = s < ns ? po[static_cast<int64_t>(s) * D] : 0.f;
    mv[i] = s < ns ? ml[2 * s] : -INFINITY;
  }
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += kMgThreads) mx = fmaxf(mx, ml[2 * s]);
  mx = wave_max64(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < kW; ++w) M = fmaxf(M, red[0][w]);
  float dsum = 0.f;
  for (int s = tid; s < ns; s += kMgThreads) dsum = fmaf(expf(ml[2 * s] - M), ml[2 * s + 1], dsum);
  dsum = wave_sum64(dsum);
  if (lane == 0) red[1][wave] = dsum;
  float num = 0.f;
#pragma unroll
  for (int i = 0; i < kPre; ++i)
    if (sl + i * kLanes < ns) num = fmaf(expf(mv[i] - M), ov[i], num);
#pragma unroll 4
  for (int s = sl + kPre * kLanes; s < ns; s += kLanes)
    num = fmaf(expf(ml[2 * s] - M), po[static_cast<int64_t>(s) * D], num);
  part[sl][c] = num;
  __syncthreads();
  if (tid < kMergeCols) {
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) den += red[1][w];
    float t = 0.f;
    for (int i = 0; i < kLanes; ++i) t += part[i][tid];
    out[bh * D + c0 + tid] = f32_to_bf16_bits(t / den);
  }
}

}  // namespace

GqaPlan gqa_plan(int B, int Hq, int Hkv, int S, bool packed) {
  constexpr int kBlock = kAtWaves * kAtPos;   // one stage per wave
  const int per_wg = packed ? Hq / Hkv : 1;
  const int64_t blocks = static_cast<int64_t>(B) * (Hq / per_wg) * div_up(S, kBlock);
  int64_t nsub = blocks / kAtTarget;
  nsub = nsub < 1 ? 1 : (nsub > 64 ? 64 : nsub);
  GqaPlan p;
  p.heads_per_wg = per_wg;
  p.rows_per_split = static_cast<int>(nsub) * kBlock;
  p.n_splits = static_cast<int>(div_up(S, p.rows_per_split));
  return p;
}

size_t gqa_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
  const GqaPlan p = gqa_plan(B, Hq, Hkv, S, true);   // the packed form has the most ranges
  return static_cast<size_t>(B) * Hq * p.n_splits * (D + 2) * sizeof(float);
}

hipError_t launch_gqa_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* lens, int B,
                             int Hq, int Hkv, int D, int S, float scale, bool packed, uint16_t* out, void* workspace,
                             hipStream_t s) {
  const GqaPlan p = gqa_plan(B, Hq, Hkv, S, packed);
  const GqaPlan pw = gqa_plan(B, Hq, Hkv, S, true);
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + static_cast<size_t>(B) * Hq * pw.n_splits * D;
  dim3 grid(static_cast<unsigned>(p.n_splits), static_cast<unsigned>(Hq / p.heads_per_wg), static_cast<unsigned>(B));
  switch (D) {
    case 64:
      hipLaunchKernelGGL(k_gqa_partial<64>, grid, dim3(kAtThreads), 0, s, q, kc, vc, lens, Hq, Hkv, S,
                         p.heads_per_wg, p.rows_per_split, p.n_splits, scale, part_o, part_ml);
      break;
    case 128:
      hipLaunchKernelGGL(k_gqa_partial<128>, grid, dim3(kAtThreads), 0, s, q, kc, vc, lens, Hq, Hkv, S,
                         p.heads_per_wg, p.rows_per_split, p.n_splits, scale, part_o, part_ml);
      break;
    default:
      hipLaunchKernelGGL(k_gqa_partial<256>, grid, dim3(kAtThreads), 0, s, q, kc, vc, lens, Hq, Hkv, S,
                         p.heads_per_wg, p.rows_per_split, p.n_splits, scale, part_o, part_ml);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gqa_merge, dim3(static_cast<unsigned>(D / kMergeCols), static_cast<unsigned>(Hq),
                                      static_cast<unsigned>(B)),
                     dim3(kMgThreads), 0, s, part_o, part_ml, lens, Hq, S, D, p.rows_per_split, p.n_splits, out);
  return hipGetLastError();
}

}  // namespace moe
