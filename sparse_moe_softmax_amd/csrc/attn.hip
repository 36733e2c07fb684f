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
// all the group's query heads (at most 8).  It stages 32 key and value rows at
// a time in LDS with 16-byte loads (the next 32 rows are loaded into registers
// meanwhile), scores every staged row against every query head (lane =
// (position, one of the wave's two heads): one dot product per lane), keeps a
// running maximum and sum per head (online softmax), and accumulates the
// weighted value rows in fp32 registers (lane = 8 columns x a group of heads;
// the four waves take every fourth position and are added at the end).  Each range leaves its (maximum, sum, unnormalised output) in
// the workspace; k_gqa_merge combines a head's ranges in range order, so the
// result does not depend on scheduling.  With one query head per workgroup
// (pack_heads == 0) the same kernel reads each key/value row once per query
// head: the unpacked form the packing is measured against.

#include "internal.hpp"
#include "attn.hpp"

namespace moe {

namespace {

constexpr int kAtSub = 32;        // positions staged per step: one per lane of a half wave
constexpr int kAtThreads = 256;
constexpr int kMgThreads = 256;   // merge
constexpr int kAtGroup = 8;       // query heads per workgroup at most
constexpr int kAtTarget = 512;    // workgroups wanted per launch (three fit a CU: 38 KB LDS, 148 VGPRs)

template <int D>
struct AttnLds {
  uint32_t q[kAtGroup][D / 2];          // query rows, bf16 pairs
  uint16_t k[kAtSub][D + 8];            // key rows; +16 bytes per row: rows start 4 banks apart
  uint16_t v[kAtSub][D];                // value rows
  float p[kAtSub][kAtGroup];            // exp(score - running max), position-major
  float alpha[kAtGroup];                // rescale of the running output for this step
};

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

__device__ inline float dot8(const uint4 a, const uint4 b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), c, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), c, false);
}

template <int D>
__global__ __launch_bounds__(kAtThreads) void k_gqa_partial(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ kc,
                                                            const uint16_t* __restrict__ vc,
                                                            const int32_t* __restrict__ lens, int Hq, int Hkv, int S,
                                                            int gw, int rows_per_split, int n_splits, float scale,
                                                            float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) AttnLds<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, b = blockIdx.z;
  const int h0 = blockIdx.y * gw;                 // first query head of this workgroup
  const int kv = h0 / (Hq / Hkv);
  const int L = min(max(lens[b], 0), S);
  const int start = split * rows_per_split;
  if (start >= L) return;                         // the merge reads only ranges below L
  const int end = min(start + rows_per_split, L);

  const uint32_t* q32 = reinterpret_cast<const uint32_t*>(q);
  for (int i = tid; i < kAtGroup * (D / 2); i += kAtThreads) {
    const int g = i / (D / 2), c = i % (D / 2);
    sm.q[g][c] = g < gw ? q32[((static_cast<int64_t>(b) * Hq + h0 + g) * D) / 2 + c] : 0u;
  }
  const int64_t row0 = (static_cast<int64_t>(b) * Hkv + kv) * S;   // cache row of position 0
  constexpr int kPieces = D / 8;                                     // 16-byte pieces per row
  constexpr int kLoads = kAtSub * kPieces / kAtThreads;              // per thread and step, each of K and V

  // score roles: lane = position within the step, wave w = query slots 2w and 2w + 1
  const int ga = 2 * wave, gb = 2 * wave + 1;
  const bool use_a = ga < gw, use_b = gb < gw;
  float m_a = -INFINITY, m_b = -INFINITY, l_a = 0.f, l_b = 0.f;

  // value roles: lane = (8-column block cb, slot group hgp); wave w takes positions w, w + 4, ...
  constexpr int kCB = D / 8;
  constexpr int kHG = 64 / kCB;      // 2, 4 or 8 slot groups
  constexpr int kHPT = kAtGroup / kHG;   // 4, 2 or 1 slots per lane
  const int cb = lane % kCB, hgp = lane / kCB;
  float acc[kHPT][8];
#pragma unroll
  for (int j = 0; j < kHPT; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[j][c] = 0.f;

  // next step's rows, loaded into registers while the current step computes
  uint4 kr[kLoads], vr[kLoads];
  auto load_step = [&](int p0) {
    const int n = min(kAtSub, end - p0);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = tid + i * kAtThreads;
      const int r = idx / kPieces, c = idx % kPieces;
      kr[i] = vr[i] = uint4{0u, 0u, 0u, 0u};
      if (r < n) {
        const int64_t off = (row0 + p0 + r) * D + c * 8;
        kr[i] = *reinterpret_cast<const uint4*>(kc + off);
        vr[i] = *reinterpret_cast<const uint4*>(vc + off);
      }
    }
  };
  load_step(start);

  for (int p0 = start; p0 < end; p0 += kAtSub) {
    const int n = min(kAtSub, end - p0);
    __syncthreads();   // the previous step's reads of k, v, p and alpha are done
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = tid + i * kAtThreads;
      const int r = idx / kPieces, c = idx % kPieces;
      *reinterpret_cast<uint4*>(&sm.k[r][c * 8]) = kr[i];
      *reinterpret_cast<uint4*>(&sm.v[r][c * 8]) = vr[i];
    }
    __syncthreads();
    if (p0 + kAtSub < end) load_step(p0 + kAtSub);

    // lane = (position lane % 32, slot 2w + lane / 32): one dot product per lane
    const int pos = lane & 31, g = 2 * wave + (lane >> 5);
    if (use_a) {   // wave-uniform
      float sa = 0.f;
      const uint16_t* krow = &sm.k[pos][0];
#pragma unroll 4
      for (int d = 0; d < D; d += 8)
        sa = dot8(*reinterpret_cast<const uint4*>(&sm.q[g][d / 2]), *reinterpret_cast<const uint4*>(krow + d), sa);
      const bool live = pos < n;
      const float sc = live ? sa * scale : -INFINITY;
      float mx = sc;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float mo = (lane >> 5) ? m_b : m_a;
      const float mn = fmaxf(mo, mx);   // finite: position 0 is live
      const float al = expf(mo - mn);
      const float e = live ? expf(sc - mn) : 0.f;
      float es = e;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) es += __shfl_xor(es, o);
      // both halves' running values, kept in every lane
      const float al_a = __shfl(al, 0), al_b = __shfl(al, 32);
      const float es_a = __shfl(es, 0), es_b = __shfl(es, 32);
      const float mn_a = __shfl(mn, 0), mn_b = __shfl(mn, 32);
      l_a = l_a * al_a + es_a;
      m_a = mn_a;
      if (use_b) {
        l_b = l_b * al_b + es_b;
        m_b = mn_b;
      }
      if (g < gw) {
        sm.p[pos][g] = e;
        if (pos == 0) sm.alpha[g] = al;
      }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      const int g = hgp * kHPT + j;
      const float al = g < gw ? sm.alpha[g] : 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[j][c] *= al;
    }
    for (int r = wave; r < n; r += 4) {
      float vf[8];
      const uint4 w = *reinterpret_cast<const uint4*>(&sm.v[r][cb * 8]);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[2 * i] = __uint_as_float(u[i] << 16);
        vf[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
      float pr[kHPT];
      if constexpr (kHPT == 4) {
        const float4 t = *reinterpret_cast<const float4*>(&sm.p[r][hgp * 4]);
        pr[0] = t.x; pr[1] = t.y; pr[2] = t.z; pr[3] = t.w;
      } else if constexpr (kHPT == 2) {
        const float2 t = *reinterpret_cast<const float2*>(&sm.p[r][hgp * 2]);
        pr[0] = t.x; pr[1] = t.y;
      } else {
        pr[0] = sm.p[r][hgp];
      }
#pragma unroll
      for (int j = 0; j < kHPT; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[j][c] = fmaf(pr[j], vf[c], acc[j][c]);
    }
  }

  // the four waves' partial sums, added in wave order, through the key and value area
  __syncthreads();
  float* red = reinterpret_cast<float*>(&sm.k[0][0]);   // [4][64][kHPT * 8]
  static_assert(4 * 64 * kHPT * 8 * sizeof(float) <= sizeof(sm.k) + sizeof(sm.v), "reduction buffer");
#pragma unroll
  for (int j = 0; j < kHPT; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) red[(wave * 64 + lane) * (kHPT * 8) + j * 8 + c] = acc[j][c];
  __syncthreads();
  for (int o = tid; o < kAtGroup * D; o += kAtThreads) {
    const int g = o / D, d = o % D;
    if (g >= gw) continue;
    const int ln = (g / kHPT) * kCB + d / 8, slot = (g % kHPT) * 8 + d % 8;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) sum += red[(w * 64 + ln) * (kHPT * 8) + slot];
    part_o[((static_cast<int64_t>(b) * Hq + h0 + g) * n_splits + split) * D + d] = sum;
  }
  if (lane == 0) {
    if (use_a) {
      float* ml = part_ml + ((static_cast<int64_t>(b) * Hq + h0 + ga) * n_splits + split) * 2;
      ml[0] = m_a;
      ml[1] = l_a;
    }
    if (use_b) {
      float* ml = part_ml + ((static_cast<int64_t>(b) * Hq + h0 + gb) * n_splits + split) * 2;
      ml[0] = m_b;
      ml[1] = l_b;
    }
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
  const int per_wg = packed ? Hq / Hkv : 1;
  const int64_t steps = static_cast<int64_t>(B) * (Hq / per_wg) * div_up(S, kAtSub);
  int64_t nsub = steps / kAtTarget;
  nsub = nsub < 1 ? 1 : (nsub > 16 ? 16 : nsub);
  GqaPlan p;
  p.heads_per_wg = per_wg;
  p.rows_per_split = static_cast<int>(nsub) * kAtSub;
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
