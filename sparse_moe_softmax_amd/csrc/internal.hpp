// Internal declarations shared by the HIP translation units of libmoe.
// Written for gfx950 (CDNA4): 64-lane wavefronts, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ vector types

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Tile height of the grouped GEMMs (rows of one block-map entry).  128 rows
// (four 32-row MFMA sub-tiles) is the most two workgroups per CU fit in
// registers and LDS.
#ifndef MOE_BM
#define MOE_BM 128
#endif
constexpr int kBM = MOE_BM;
static_assert(kBM % 32 == 0, "tile height: whole 32-row MFMA sub-tiles");
constexpr int kTopkTile = 16;       // tokens per routing tile (histogram granularity)

// ------------------------------------------------------------------ scalar helpers

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // one v_cvt_pk_bf16_f32: round-to-nearest-even of both values
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline uint16_t f32_to_bf16_bits(float v) { return static_cast<uint16_t>(pack_bf16x2(v, 0.f)); }

// Dequantise the 8 int4 codes of one dword (element i in nibble i, low nibble
// first) to 8 bf16 values w = bf16_rne(c*s + b), returned as 4 packed dwords
// (element 2j in the low half of dword j).
//
// Each nibble is isolated into a 16-bit half, where as an fp16 bit pattern it
// is the subnormal c*2^-24 (nibbles 0, 2) or c*2^-20 (nibbles 1, 3 of a byte
// pair, left in place x16); v_fma_mix_f32 widens the half exactly and computes
// c*(s*2^24)*2^-24 + b with a single rounding of an exact value, i.e. the fp32
// value c*s + b (c*s is exact in fp32: a 4-bit by 11-bit product).
__device__ inline uint4 dequant8(uint32_t q, float s24, float s20, float bias) {
  const uint32_t t0 = q & 0x000F000Fu;          // elements 0 | 4
  const uint32_t t1 = q & 0x00F000F0u;          // elements 1 | 5   (x16)
  const uint32_t qs = q >> 8;
  const uint32_t t2 = qs & 0x000F000Fu;         // elements 2 | 6
  const uint32_t t3 = qs & 0x00F000F0u;         // elements 3 | 7   (x16)
  const f16x2 h0 = __builtin_bit_cast(f16x2, t0);
  const f16x2 h1 = __builtin_bit_cast(f16x2, t1);
  const f16x2 h2 = __builtin_bit_cast(f16x2, t2);
  const f16x2 h3 = __builtin_bit_cast(f16x2, t3);
  const float v0 = __builtin_fmaf(static_cast<float>(h0.x), s24, bias);
  const float v4 = __builtin_fmaf(static_cast<float>(h0.y), s24, bias);
  const float v1 = __builtin_fmaf(static_cast<float>(h1.x), s20, bias);
  const float v5 = __builtin_fmaf(static_cast<float>(h1.y), s20, bias);
  const float v2 = __builtin_fmaf(static_cast<float>(h2.x), s24, bias);
  const float v6 = __builtin_fmaf(static_cast<float>(h2.y), s24, bias);
  const float v3 = __builtin_fmaf(static_cast<float>(h3.x), s20, bias);
  const float v7 = __builtin_fmaf(static_cast<float>(h3.y), s20, bias);
  uint4 r;
  r.x = pack_bf16x2(v0, v1);
  r.y = pack_bf16x2(v2, v3);
  r.z = pack_bf16x2(v4, v5);
  r.w = pack_bf16x2(v6, v7);
  return r;
}

// Per-group constants for dequant8 from fp16 scale / bias bit patterns.
struct DqConst {
  float s24, s20, bias;
};
__device__ inline DqConst dq_const(uint16_t scale_bits, uint16_t bias_bits) {
  const float s = static_cast<float>(__builtin_bit_cast(_Float16, scale_bits));
  DqConst c;
  c.s24 = s * 16777216.0f;  // exact: power-of-two scaling
  c.s20 = s * 1048576.0f;
  c.bias = static_cast<float>(__builtin_bit_cast(_Float16, bias_bits));
  return c;
}

__device__ inline f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ direct-to-LDS loads

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global -> LDS loads through buffer instructions.  Lane i of the wave
// writes its bytes at lds + i * 16 (16-byte form) or lds + i * 4 (4-byte form);
// the source is the resource's base + a per-lane offset + a wave-uniform offset,
// so that advancing a stream by one K block is a scalar add.  Issued through
// inline asm so that the compiler does not add its own conservative vmcnt(0)
// wait before every later LDS read: the K loop waits for exactly the stage it
// consumes (wait_vmcnt) and then barriers.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// Raw buffer resource at `base` covering the whole 32-bit offset range
// (num_records all ones: no range clamp; offsets are in bytes).
__device__ inline i32x4 buffer_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(a));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(a >> 32));  // stride 0
  r.z = -1;
  r.w = 0x00020000;
  return r;
}
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ inline void bdma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               : : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ inline void bdma4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               : : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
// vmcnt(n * per) for a runtime n in [0, MAXN] (s_waitcnt takes an immediate).
template <int PER, int MAXN>
__device__ inline void wait_stages(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt<MAXN * PER>();
      return;
    }
    wait_stages<PER, MAXN - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// Physical 16-byte chunk of logical chunk c in row r of an A stage.  The XOR
// key (r ^ (r >> 3)) & 7 makes the 16-byte reads of any 8 consecutive rows, and
// of the even and of the odd rows among any 16 consecutive rows, hit distinct
// bank groups (conflict-free for 32- and 64-bank LDS).
__device__ inline int a_chunk(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }
// ------------------------------------------------------------------ top-k (device helpers)

// Order-preserving 32-bit key of a logit (-0 folded onto +0): larger logit,
// larger key; equal logits, equal keys.
__device__ inline uint32_t topk_key32(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float topk_key32_value(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
}
// max over a 16-lane DPP row (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror): afterwards every lane of the row holds it
__device__ inline uint32_t row_max16_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  return max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
}

// Top-k (k <= 16) of E <= 256 logits by one whole wave: lane l holds experts
// l, l + 64, l + 128, l + 192.  Order: larger logit first, then lower expert
// index (-0 and +0 tie).  Each of the k rounds finds the largest
// remaining 32-bit key (per-lane max, DPP row max, max of the four rows in
// scalar registers); among the lanes holding it, the lowest expert index wins
// (the first slot i whose ballot is non-empty, then its lowest lane), and that
// one entry is removed (key 0: real keys are >= 1).  Results are the same in
// every lane.  v[i]: logit of expert lane + 64 i (ignored for experts >= E).
__device__ inline void topk_wave64_regs(const float (&v)[4], int E, int k, int (&top_e)[16], float (&top_v)[16]) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = lane + 64 * i < E ? topk_key32(v[i]) : 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < k) {
      uint32_t m = max(max(key[0], key[1]), max(key[2], key[3]));
      m = row_max16_u32(m);
      uint32_t best = __builtin_amdgcn_readlane(m, 0);
      best = max(best, static_cast<uint32_t>(__builtin_amdgcn_readlane(m, 16)));
      best = max(best, static_cast<uint32_t>(__builtin_amdgcn_readlane(m, 32)));
      best = max(best, static_cast<uint32_t>(__builtin_amdgcn_readlane(m, 48)));
      int e = 0;
      bool found = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t bal = __ballot(key[i] == best);
        if (!found && bal != 0) {
          e = 64 * i + static_cast<int>(__builtin_ctzll(bal));
          found = true;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) key[i] = (lane + 64 * i == e) ? 0u : key[i];
      top_e[r] = e;
      top_v[r] = topk_key32_value(best);
    }
  }
}
// The same with the logits in memory (LDS).
__device__ inline void topk_wave64(const float* __restrict__ logits, int E, int k, int (&top_e)[16],
                                   float (&top_v)[16]) {
  const int lane = threadIdx.x & 63;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = lane + 64 * i < E ? logits[lane + 64 * i] : 0.f;
  topk_wave64_regs(v, E, k, top_e, top_v);
}

// Renormalised weights of the k kept experts: exp(l_r - l_0) / sum_r' exp(l_r' - l_0),
// summed in slot order.
__device__ inline void topk_weights(int k, const float (&top_v)[16], float (&w)[16]) {
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < k) {
      w[r] = expf(top_v[r] - top_v[0]);
      sum += w[r];
    }
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (r < k) w[r] = w[r] * inv;
}

__device__ inline float sigmoidf_(float s) { return 1.0f / (1.0f + expf(-s)); }

// ------------------------------------------------------------------ launch helpers (host)

struct GemmTiles {
  const int32_t* perm;       // grouped position -> flat slot (routed tiles)
  const int32_t* offsets;    // [E+1]
  const int32_t* block_map;  // [max_tiles][2]
  const int32_t* n_tiles;    // device scalar
  int32_t max_tiles;         // routed tile bound (grid sizing)
  int32_t block_m;           // rows per routed tile (<= kBM)
  int32_t n_shared_chunks;   // shared-expert tiles of kBM rows put first (0 = none)
  const int32_t* tile_rows;  // [max_tiles] rows of each routed tile, or NULL: from offsets
};

// Geometry of the packed (matrix-core) layout of one expert matrix: slices of
// 256 product columns x K blocks of 64, 9216 bytes per (slice, K block).
struct PackGeom {
  int N, K, Iw;       // canonical rows, reduction length, SwiGLU width (gate/up kinds)
  int slices, kg;     // slices per expert, K blocks
  bool swiglu;        // gate/up column order (32 gate + 32 up per wave)
  int64_t expert_bytes;
};
inline PackGeom pack_geom(const moe_dims& d, int matrix) {
  PackGeom g{};
  const bool sh = matrix == MOE_MAT_SH_GATE_UP || matrix == MOE_MAT_SH_DOWN;
  g.Iw = sh ? d.shared_inter : d.inter;
  g.swiglu = matrix == MOE_MAT_GATE_UP || matrix == MOE_MAT_SH_GATE_UP;
  if (g.swiglu) {
    g.N = 2 * g.Iw;
    g.K = d.hidden;
    g.slices = static_cast<int>((g.Iw + 127) / 128);
  } else {
    g.N = d.hidden;
    g.K = g.Iw;
    g.slices = static_cast<int>((d.hidden + 255) / 256);
  }
  g.kg = g.K / 64;
  g.expert_bytes = static_cast<int64_t>(g.slices) * g.kg * 9216;
  return g;
}

hipError_t launch_prepack_q4(const moe_dims& d, int matrix, const moe_q4& w, int n_exp, uint8_t* packed,
                             hipStream_t s);
hipError_t launch_prepack_router(const float* w, uint16_t* w3, int E, int H, hipStream_t s);
// Router GEMM with K split over `splits` workgroups (splits divides H/64).
// splits == 1: out = logits (+ bias), s_out = shared logit (NULL to skip).
// splits > 1: out = partial sums [splits][T][E], s_out = [splits][T], no bias.
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w3, const float* bias, const float* wsg, int T,
                              int H, int E, int splits, float* out, float* s_out, hipStream_t s);
// K splits the fused layer uses for T tokens (enough workgroups to fill the chip).
int router_splits(int T, int H, int E);
hipError_t launch_router_gemv(const uint16_t* x, const float* w, const float* bias, const float* wsg, int T, int H,
                              int E, float* logits, float* s_logit, hipStream_t s);
// Top-k from router output: splits == 1 reads final logits (and shared logit);
// splits > 1 sums the partials in split order, adds the bias and writes the
// final logits / shared logit to logits_out / s_out when given.
hipError_t launch_topk(const float* parts, const float* s_parts, int splits, const float* bias, int T, int E, int k,
                       float* logits_out, float* s_out, int32_t* ids, float* wts, float* gate, int32_t* tilehist,
                       hipStream_t s);
// err (nullable): device error word; ids outside [0, E) set MOE_DEVERR_EXPERT_ID and are skipped.
hipError_t launch_tile_hist(const int32_t* ids, int T, int k, int E, int32_t* tilehist, uint32_t* err, hipStream_t s);
// The two halves of launch_group: per-expert counts (and per-tile bases), then
// offsets + permutation (+ block map and n_tiles when write_map).
hipError_t launch_group_counts(const int32_t* tilehist, int32_t* tilebase, int T, int E, int32_t* counts,
                               hipStream_t s);
// tile_rows (nullable): rows of each tile of the block map, written in either case.
hipError_t launch_group_scatter(const int32_t* ids, const int32_t* counts, const int32_t* tilebase, int T, int k,
                                int E, int block_m, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* block_map, int max_tiles, int32_t* n_tiles, bool write_map,
                                int32_t* tile_rows, uint32_t* err, hipStream_t s);
hipError_t launch_group(const int32_t* ids, const int32_t* tilehist, int32_t* tilebase, int T, int k, int E,
                        int block_m, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* block_map, int max_tiles, int32_t* n_tiles, int32_t* tile_rows, uint32_t* err,
                        hipStream_t s);
// gather: routed A rows are token rows a[perm[p] / k] (else grouped rows a[p]).
hipError_t launch_gemm_swiglu(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* x,
                              bool gather, const GemmTiles& tl, int T, uint16_t* h, uint16_t* h_sh, hipStream_t s);
hipError_t launch_gemm_scatter(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                               bool gather, const uint16_t* h_sh, const GemmTiles& tl, const float* row_w,
                               const float* gate, int T, float* y, hipStream_t s);
// Down GEMM writing every slot's unweighted output, slot[t][j][:] (routed j < k,
// shared j = k), as fp16 with a power-of-two exponent per 64 columns in
// slot_exp [T][k+1][H/64].
hipError_t launch_gemm_slots(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                             const uint16_t* h_sh, const GemmTiles& tl, int T, uint16_t* slots, uint8_t* slot_exp,
                             hipStream_t s);
// out[t] = bf16( sum_{j<k} w[t][j] * o_j + gate[t] * o_k ) in slot order, o_j the
// slot values times 2^exponent (w or gate NULL = 1).
hipError_t launch_combine(const uint16_t* slots, const uint8_t* slot_exp, const float* w, const float* gate,
                          uint16_t* out, int T, int H, int k, hipStream_t s);
struct DecodePtrs {
  float* logits;
  float* s_logit;
  int32_t* ids;
  float* wts;
  float* gate;
  void* sync;        // decode_sync_bytes(), zero before the first call on it
  uint32_t* err;     // device error word (MOE_DEVERR_* bits)
};
// The whole layer for 1 <= T <= kDecMaxT tokens as one launch (router, top-k,
// experts, combine), where decode_supported(d, T).
constexpr int kDecMaxT = 4;
hipError_t launch_decode_layer(const moe_dims& d, const moe_layer& L, const uint16_t* x, int T, uint16_t* y,
                               const DecodePtrs& p, hipStream_t s);
bool decode_supported(const moe_dims& d, int T);
// Workgroups the fused layer for (d, T) launches, and how many of its
// workgroups the current device holds at once.
hipError_t decode_residency(const moe_dims& d, int T, int* needed, int* resident);
size_t decode_sync_bytes(const moe_dims& d);

__host__ __device__ inline int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
