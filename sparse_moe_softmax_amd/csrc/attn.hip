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
// all the group's query heads (at most 8).  It stages 64 key and value rows at
// a time in LDS with 16-byte loads, scores every staged row against every
// query head (lane = position, wave = two heads), keeps a running maximum and
// sum per head (online softmax), and accumulates the weighted value rows in
// fp32 registers.  Each range leaves its (maximum, sum, unnormalised output) in
// the workspace; k_gqa_merge combines a head's ranges in range order, so the
// result does not depend on scheduling.  With one query head per workgroup
// (pack_heads == 0) the same kernel reads each key/value row once per query
// head: the unpacked form the packing is measured against.

#include "internal.hpp"

namespace moe {

namespace {

constexpr int kAtSub = 64;        // positions staged per step
constexpr int kAtThreads = 256;
constexpr int kAtGroup = 8;       // query heads per workgroup at most
constexpr int kAtTarget = 512;    // workgroups wanted per launch (two per CU)

template <int D>
struct AttnLds {
  float q[kAtGroup][D];                 // query rows, fp32
  uint16_t k[kAtSub][D + 8];            // key rows; +16 bytes per row: rows start 4 banks apart
  uint16_t v[kAtSub][D];                // value rows
  float p[kAtGroup][kAtSub];            // exp(score - running max)
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

__device__ inline void unpack8(const uint4 w, float* f) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
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

  for (int i = tid; i < kAtGroup * D; i += kAtThreads) {
    const int g = i / D, d = i % D;
    sm.q[g][d] = g < gw ? bf16_to_f32(q[(static_cast<int64_t>(b) * Hq + h0 + g) * D + d]) : 0.f;
  }
  const int64_t row0 = (static_cast<int64_t>(b) * Hkv + kv) * S;   // cache row of position 0
  constexpr int kPieces = D / 8;                                     // 16-byte pieces per row

  // score roles: lane = position within the step, wave w = query slots 2w and 2w + 1
  const int ga = 2 * wave, gb = 2 * wave + 1;
  const bool use_a = ga < gw, use_b = gb < gw;
  float m_a = -INFINITY, m_b = -INFINITY, l_a = 0.f, l_b = 0.f;

  // value roles: thread = (column pair, group of query slots)
  constexpr int kPairs = D / 2;
  constexpr int kHg = kAtThreads / kPairs;   // 2, 4 or 8 slot groups
  constexpr int kHpt = kAtGroup / kHg;       // 4, 2 or 1 slots per thread
  const int cp = tid % kPairs, hg = tid / kPairs;
  float acc[kHpt][2];
#pragma unroll
  for (int j = 0; j < kHpt; ++j) acc[j][0] = acc[j][1] = 0.f;

  for (int p0 = start; p0 < end; p0 += kAtSub) {
    const int n = min(kAtSub, end - p0);
    __syncthreads();   // the previous step's reads of k, v, p and alpha are done
    for (int i = tid; i < kAtSub * kPieces; i += kAtThreads) {
      const int r = i / kPieces, c = i % kPieces;
      uint4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (r < n) {
        const int64_t off = (row0 + p0 + r) * D + c * 8;
        kw = *reinterpret_cast<const uint4*>(kc + off);
        vw = *reinterpret_cast<const uint4*>(vc + off);
      }
      *reinterpret_cast<uint4*>(&sm.k[r][c * 8]) = kw;
      *reinterpret_cast<uint4*>(&sm.v[r][c * 8]) = vw;
    }
    __syncthreads();

    if (use_a) {   // wave-uniform
      float sa = 0.f, sb = 0.f;
      const uint16_t* kr = &sm.k[lane][0];
#pragma unroll 4
      for (int d = 0; d < D; d += 8) {
        float kf[8];
        unpack8(*reinterpret_cast<const uint4*>(kr + d), kf);
        const float4 qa0 = *reinterpret_cast<const float4*>(&sm.q[ga][d]);
        const float4 qa1 = *reinterpret_cast<const float4*>(&sm.q[ga][d + 4]);
        const float4 qb0 = *reinterpret_cast<const float4*>(&sm.q[gb][d]);
        const float4 qb1 = *reinterpret_cast<const float4*>(&sm.q[gb][d + 4]);
        sa = fmaf(qa0.x, kf[0], sa); sa = fmaf(qa0.y, kf[1], sa); sa = fmaf(qa0.z, kf[2], sa);
        sa = fmaf(qa0.w, kf[3], sa); sa = fmaf(qa1.x, kf[4], sa); sa = fmaf(qa1.y, kf[5], sa);
        sa = fmaf(qa1.z, kf[6], sa); sa = fmaf(qa1.w, kf[7], sa);
        sb = fmaf(qb0.x, kf[0], sb); sb = fmaf(qb0.y, kf[1], sb); sb = fmaf(qb0.z, kf[2], sb);
        sb = fmaf(qb0.w, kf[3], sb); sb = fmaf(qb1.x, kf[4], sb); sb = fmaf(qb1.y, kf[5], sb);
        sb = fmaf(qb1.z, kf[6], sb); sb = fmaf(qb1.w, kf[7], sb);
      }
      const bool live = lane < n;
      {
        const float s = live ? sa * scale : -INFINITY;
        const float mn = fmaxf(m_a, wave_max64(s));   // finite: lane 0 is live
        const float al = expf(m_a - mn);
        const float e = live ? expf(s - mn) : 0.f;
        l_a = l_a * al + wave_sum64(e);
        m_a = mn;
        sm.p[ga][lane] = e;
        if (lane == 0) sm.alpha[ga] = al;
      }
      if (use_b) {
        const float s = live ? sb * scale : -INFINITY;
        const float mn = fmaxf(m_b, wave_max64(s));
        const float al = expf(m_b - mn);
        const float e = live ? expf(s - mn) : 0.f;
        l_b = l_b * al + wave_sum64(e);
        m_b = mn;
        sm.p[gb][lane] = e;
        if (lane == 0) sm.alpha[gb] = al;
      }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < kHpt; ++j) {
      const int g = hg * kHpt + j;
      if (g < gw) {
        const float al = sm.alpha[g];
        acc[j][0] *= al;
        acc[j][1] *= al;
      }
    }
    for (int r = 0; r < n; ++r) {
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(&sm.v[r][2 * cp]);
      const float v0 = __uint_as_float(vv << 16), v1 = __uint_as_float(vv & 0xffff0000u);
#pragma unroll
      for (int j = 0; j < kHpt; ++j) {
        const int g = hg * kHpt + j;
        if (g < gw) {
          const float pr = sm.p[g][r];
          acc[j][0] = fmaf(pr, v0, acc[j][0]);
          acc[j][1] = fmaf(pr, v1, acc[j][1]);
        }
      }
    }
  }

#pragma unroll
  for (int j = 0; j < kHpt; ++j) {
    const int g = hg * kHpt + j;
    if (g < gw) {
      float* o = part_o + ((static_cast<int64_t>(b) * Hq + h0 + g) * n_splits + split) * D + 2 * cp;
      *reinterpret_cast<float2*>(o) = make_float2(acc[j][0], acc[j][1]);
    }
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

// One workgroup per (query head, sequence): the ranges' partial results in
// range order, out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, rounded to bf16.
__global__ __launch_bounds__(kAtThreads) void k_gqa_merge(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int32_t* __restrict__ lens, int Hq, int S, int D,
                                                          int rows_per_split, int n_splits, uint16_t* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(lens[b], 0), S);
  const int ns = (L + rows_per_split - 1) / rows_per_split;
  const int64_t bh = static_cast<int64_t>(b) * Hq + h;
  const float* ml = part_ml + bh * n_splits * 2;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float den = 0.f;
  for (int s = 0; s < ns; ++s) den = fmaf(expf(ml[2 * s] - M), ml[2 * s + 1], den);
  for (int d = threadIdx.x; d < D; d += kAtThreads) {
    float num = 0.f;
    for (int s = 0; s < ns; ++s) num = fmaf(expf(ml[2 * s] - M), part_o[(bh * n_splits + s) * D + d], num);
    out[bh * D + d] = ns ? f32_to_bf16_bits(num / den) : static_cast<uint16_t>(0);
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
  hipLaunchKernelGGL(k_gqa_merge, dim3(static_cast<unsigned>(Hq), static_cast<unsigned>(B)), dim3(kAtThreads), 0, s,
                     part_o, part_ml, lens, Hq, S, D, p.rows_per_split, p.n_splits, out);
  return hipGetLastError();
}

}  // namespace moe
