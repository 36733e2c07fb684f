// Vector-ALU building blocks of the matrix-vector (decode) path.  With one or
// a few tokens, each touched expert's weights are used once per token, so the
// work is matrix-vector,
// bound by memory, and done on the vector ALUs rather than the matrix units
// (Lily page, section "Why Apple Silicon isn't just a smaller datacenter
// GPU").  Weights are read in the canonical row-major int4 layout, one row
// being one coalesced read across the wave, and dequantised in registers
// exactly as in the grouped GEMM: bf16 of the exact fp32 c*s + b, multiplied
// with v_dot2_f32_bf16.
#pragma once
#include "internal.hpp"

namespace moe {

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

template <int kCtrl>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the wave, the same in every lane: a DPP sum within each row of 16
// lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror: every lane of a row ends with the same value), then the four row
// sums in a fixed order.  The whole wave must be active.
__device__ inline float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
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

}  // namespace moe
