// Grouped expert GEMMs with int4 weights dequantised in registers
// ("By reconstructing 4-bit weights one tile at a time within grouped GEMM
// operations, Lily keeps the expanded arrays inside GPU registers": Inside
// Lily page, section "Performance Gains and Workload Patterns"; prefill work
// is matrix-matrix and belongs on the matrix units: Lily page, section "Why
// Apple Silicon isn't just a smaller datacenter GPU").
//
// Work unit (workgroup of 4 waves) = one tile of up to kBM rows of one expert
// x one slice of 256 weight rows (product columns).  Tiles come from the block
// map (routed experts) and, in the fused layer, from kBM-row chunks of the
// shared expert, which are placed first (the largest tiles start first).
//
// Data path per 64-wide K block ("stage"), all asynchronous:
//   * global -> LDS direct loads (global_load_lds, no register staging) of
//       - the tile's activation rows, bf16 [kBM][64], rows gathered through the
//         permutation; 16-byte chunks XOR-swizzled by row so that MFMA
//         fragment reads are bank-conflict free without padding,
//       - the slice's int4 codes [256 rows][32 B] and fp16 scales and biases;
//   * a ring of kStages stages in LDS, refilled kStages-1 blocks ahead, with
//     explicit vmcnt waits (every vector-memory instruction inside the loop is
//     one of these loads, issued in a fixed order and count per stage) and one
//     barrier per K block;
//   * each wave reads its 64 columns' codes from LDS and dequantises them in
//     registers into MFMA B fragments: exact fp32 c*s + b, one nearest-even
//     rounding to bf16 (see dequant8).  Dequantised weights never reach LDS or HBM;
//   * all A fragments of the block are loaded into registers first; then for
//     each of the 4 column groups the B fragment is built and used by every
//     row sub-tile, so the VALU work of the next group overlaps the MFMAs of
//     the current one (v_mfma_f32_16x16x32_bf16, fp32 accumulators).
// Inside a K block of 64 the lane group q = lane/16 covers K offsets
// [16q, 16q+16) and fragment s holds 16q+8s .. +7 for both operands: a
// consistent permutation of K, which leaves the dot products unchanged.
//
// Epilogues (through LDS so that every lane stores 16 contiguous bytes):
//   SWIGLU : wave columns = 32 gate rows + the matching 32 up rows;
//            h = bf16( silu(gate) * up ) in grouped order.
//   SCATTER: y[token][col] += weight * o, fp32 atomics (standalone op).
//   SLOTS  : slot[token][j][col] = fp16(weight * o): the weighted output of
//            slot j of the token (routed: its routing weight; shared expert:
//            slot k with the sigmoid gate), token-major, for a fixed-order
//            combine afterwards.  No atomics.
//
// Launch order is XCD-aware: consecutive workgroup ids go round-robin to the 8
// XCDs, so ids are mapped such that all column slices of one tile share an XCD
// (and its L2) and consecutive tiles spread over the XCDs.
#include "internal.hpp"

namespace moe {

constexpr int kGemmThreads = 256;
constexpr int kStages = 4;
constexpr int kAStage = kBM * 128;           // bf16 [kBM][64], swizzled 16-byte chunks
constexpr int kBStage = 256 * 32;            // int4 codes of 256 weight rows x 64 K
constexpr int kSStage = 256 * 4;             // fp16 scale per row, zero-extended to 4 bytes
constexpr int kStageBytes = kAStage + kBStage + 2 * kSStage;
constexpr int kDmaPerStage = kBM / 32 + 4;   // direct loads per wave per stage
static_assert(kStageBytes * kStages <= 160 * 1024, "LDS ring too large");
static_assert((kStages - 2) * kDmaPerStage <= 63, "vmcnt range");
static_assert(kStages == 4, "the wait ladder in the K loop covers 2, 1 and 0 newer stages");

enum { kSwiglu = 0, kScatter = 1, kSlots = 2 };

struct GemmArgs {
  // index 0: routed experts, 1: shared expert
  const uint8_t* codes[2];
  const uint16_t* scales[2];
  const uint16_t* biases[2];
  int K[2];        // reduction length
  int N[2];        // weight rows per expert matrix
  int Ih[2];       // SWIGLU: intermediate width (gate rows 0..Ih-1, up rows Ih..2Ih-1)
  const uint16_t* a[2];
  int lda[2];
  void* out[2];
  int ldo[2];
  const int32_t* perm;
  const int32_t* offsets;
  const int32_t* block_map;
  const int32_t* n_tiles;
  const float* row_w;   // routed: weight per flat slot
  const float* gate;    // shared: sigmoid gate per token
  int block_m;
  int n_sh;             // shared chunks (first in the chunk order)
  int max_tiles;
  int n_slices;
  int T, k, H;
};

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global -> LDS loads.  Lane i of the wave writes its bytes at
// lds + i * 16 (16-byte form) or lds + i * 4 (2-byte form, zero-extended).
// Issued through inline asm so that the compiler does not add its own
// conservative vmcnt(0) wait before every later LDS read: the K loop waits for
// exactly the stage it consumes (wait_vmcnt) and then barriers.
__device__ inline uint32_t lds_addr(const void* p) {
  // wave-uniform by construction; readfirstlane puts it in an SGPR for M0
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
__device__ inline void dma16(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds_addr(lds)) : "memory", "m0");
}
__device__ inline void dma2(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ushort %0, off" : : "v"(g), "s"(lds_addr(lds)) : "memory", "m0");
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_q4(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStageBytes];

  // ---- which tile / slice
  const int wg = blockIdx.x;
  const int S = g.n_slices;
  const int xcd = wg & 7;
  const int rr = wg >> 3;
  const int chunk = (rr / S) * 8 + xcd;
  const int slice = rr % S;
  if (chunk >= g.n_sh + g.max_tiles) return;
  int which, e, row0, rows;
  if (chunk < g.n_sh) {
    which = 1;
    e = 0;
    row0 = chunk * kBM;
    rows = min(kBM, g.T - row0);
  } else {
    const int tile = chunk - g.n_sh;
    if (tile >= *g.n_tiles) return;
    which = 0;
    e = g.block_map[2 * tile];
    row0 = g.block_map[2 * tile + 1];
    rows = min(g.block_m, g.offsets[e + 1] - row0);
  }
  const int K = g.K[which];
  const int N = g.N[which];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int q = lane >> 4;

  // ---- the 256 weight rows of this slice; wave w owns rows [64w, 64w + 64) of it
  //      (as 4 column groups of 16), `wr(i)` maps a slice row to a matrix row.
  bool active;
  int Ih = 0, hc = 0, n0 = 0;
  if (MODE == kSwiglu) {
    Ih = g.Ih[which];
    if (slice * 128 >= Ih) return;  // whole block idle (narrower shared expert)
    hc = slice * 128 + wave * 32;
    active = hc < Ih;
  } else {
    n0 = slice * 256 + wave * 64;
    active = n0 < N;
  }
  // slice row i (0..255) -> matrix row; rows of idle waves map to row 0 (valid memory)
  auto wr = [&](int i) -> int {
    const int w = i >> 6, r = i & 63;
    if (MODE == kSwiglu) {
      const int h0 = slice * 128 + w * 32;
      if (h0 >= Ih) return 0;
      return (r < 32) ? h0 + r : Ih + h0 + (r - 32);
    }
    const int nn = slice * 256 + i;
    return (slice * 256 + w * 64 < N) ? nn : 0;
  };
  const int kg = K / 64;
  const uint8_t* cbase = g.codes[which] + static_cast<int64_t>(e) * N * (K / 2);
  const uint16_t* sbase = g.scales[which] + static_cast<int64_t>(e) * N * kg;
  const uint16_t* bbase = g.biases[which] + static_cast<int64_t>(e) * N * kg;

  // ---- per-lane sources of the direct loads (fixed for the whole K loop)
  constexpr int kAI = kBM / 32;  // A instructions per wave per stage (8 rows each)
  const uint16_t* abase = g.a[which];
  const int lda = g.lda[which];
  const uint16_t* asrc[kAI];
#pragma unroll
  for (int j = 0; j < kAI; ++j) {
    const int r = (wave * kAI + j) * 8 + (lane >> 3);   // tile row this lane fills
    const int p = lane & 7;                             // physical 16-byte chunk
    const int c = p ^ (r & 7);                          // logical chunk it holds
    int rsrc = (r < rows) ? r : 0;                      // padding rows load row 0 (ignored)
    int64_t arow;
    if (which == 1 || MODE != kSwiglu)
      arow = row0 + rsrc;
    else
      arow = g.perm[row0 + rsrc] / g.k;
    asrc[j] = abase + arow * lda + c * 8;
  }
  const uint8_t* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = wave * 64 + j * 32 + (lane >> 1);
    bsrc[j] = cbase + static_cast<int64_t>(wr(i)) * (K / 2) + (lane & 1) * 16;
  }
  const int srow = wr(wave * 64 + lane);
  const uint16_t* ssrc = sbase + static_cast<int64_t>(srow) * kg;
  const uint16_t* zsrc = bbase + static_cast<int64_t>(srow) * kg;

  auto issue = [&](int kb) {
    unsigned char* st = ring + (kb % kStages) * kStageBytes;
#pragma unroll
    for (int j = 0; j < kAI; ++j) dma16(asrc[j] + kb * 64, st + (wave * kAI + j) * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(bsrc[j] + kb * 32, st + kAStage + (wave * 64 + j * 32) * 32);
    dma2(ssrc + kb, st + kAStage + kBStage + wave * 256);
    dma2(zsrc + kb, st + kAStage + kBStage + kSStage + wave * 256);
  };

  f32x4 acc[kMSub][4];
#pragma unroll
  for (int m = 0; m < kMSub; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsub = (rows + 15) >> 4;

  // ---- prologue: stages 0 .. kStages-2 in flight
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < kg) issue(s);

  for (int kb = 0; kb < kg; ++kb) {
    // wait for this wave's loads of stage kb (newer stages may stay in flight)
    const int newer = min(kStages - 2, kg - 1 - kb);
    if (newer >= kStages - 2)
      wait_vmcnt<(kStages - 2) * kDmaPerStage>();
    else if (newer == 1)
      wait_vmcnt<kDmaPerStage>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // every wave's loads of stage kb landed; stage kb-1 fully consumed
    if (kb + kStages - 1 < kg) issue(kb + kStages - 1);

    const unsigned char* st = ring + (kb % kStages) * kStageBytes;
    if (active) {
      // A fragments of every row sub-tile
      bf16x8 af[kMSub][2];
#pragma unroll
      for (int m = 0; m < kMSub; ++m) {
        if (m < nsub) {
          const int r = m * 16 + col;
          const unsigned char* rp = st + r * 128;
          af[m][0] = *reinterpret_cast<const bf16x8*>(rp + (((2 * q) ^ (r & 7)) << 4));
          af[m][1] = *reinterpret_cast<const bf16x8*>(rp + (((2 * q + 1) ^ (r & 7)) << 4));
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = wave * 64 + c * 16 + col;
        const uint2 codes = *reinterpret_cast<const uint2*>(st + kAStage + i * 32 + q * 8);
        const uint16_t sc = *reinterpret_cast<const uint16_t*>(st + kAStage + kBStage + i * 4);
        const uint16_t bz = *reinterpret_cast<const uint16_t*>(st + kAStage + kBStage + kSStage + i * 4);
        const DqConst dc = dq_const(sc, bz);
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, dequant8(codes.x, dc.s24, dc.s20, dc.bias));
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, dequant8(codes.y, dc.s24, dc.s20, dc.bias));
#pragma unroll
        for (int m = 0; m < kMSub; ++m) {
          if (m < nsub) {
            acc[m][c] = mfma16(af[m][0], b0, acc[m][c]);
            acc[m][c] = mfma16(af[m][1], b1, acc[m][c]);
          }
        }
      }
    }
  }
  // ---- epilogue.  C fragment: lane holds rows 4q..4q+3 of a 16-row sub-tile, column `col`.
  // Each wave stages one 16-row sub-tile at a time in a private 2 KB LDS area
  // at the start of the ring, which is free once every wave has left the loop.
  __syncthreads();
  if (!active) return;
  unsigned char* stg = ring + wave * 2048;
  if (MODE == kSwiglu) {
    uint16_t* out = static_cast<uint16_t*>(g.out[which]);
    const int ldo = g.ldo[which];
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
      if (m < nsub) {
        // 16 rows x 32 h columns, bf16 (64 B per row)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float gt = acc[m][c][i];
            const float up = acc[m][c + 2][i];
            const float h = gt / (1.0f + __expf(-gt)) * up;
            reinterpret_cast<uint16_t*>(stg)[(q * 4 + i) * 32 + c * 16 + col] = f32_to_bf16_bits(h);
          }
        }
        __builtin_amdgcn_wave_barrier();
        // lane -> row lane/4, 16-byte piece lane%4
        const int r = lane >> 2, pc = lane & 3;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 64 + pc * 16);
        const int rt = m * 16 + r;
        if (rt < rows) *reinterpret_cast<uint4*>(out + static_cast<int64_t>(row0 + rt) * ldo + hc + pc * 8) = v;
        __builtin_amdgcn_wave_barrier();
      }
    }
  } else if (MODE == kSlots) {
    uint16_t* out = static_cast<uint16_t*>(g.out[0]);   // [T][k+1][H] fp16
    const int H = g.H, k = g.k;
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
      if (m < nsub) {
        float wt[4];
        int64_t orow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rt = min(m * 16 + q * 4 + i, rows - 1);
          if (which == 1) {
            const int t = row0 + rt;
            wt[i] = g.gate[t];
            orow[i] = static_cast<int64_t>(t) * (k + 1) + k;
          } else {
            const int f = g.perm[row0 + rt];
            wt[i] = g.row_w[f];
            orow[i] = static_cast<int64_t>(f / k) * (k + 1) + (f % k);
          }
        }
        // 16 rows x 64 columns, fp16 (128 B per row): two halves of 8 rows
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const _Float16 v = static_cast<_Float16>(wt[i] * acc[m][c][i]);
            reinterpret_cast<_Float16*>(stg)[(q * 4 + i) * 64 + c * 16 + col] = v;
          }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int r = half * 8 + (lane >> 3), pc = lane & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 128 + pc * 16);
          // the row's destination: held by lane with q = r/4, i = r%4
          const int rt = m * 16 + r;
          int64_t dst;
          {
            const int src_lane = (r >> 2) * 16;
            const int ii = r & 3;
            int64_t o0 = __shfl(orow[0], src_lane), o1 = __shfl(orow[1], src_lane);
            int64_t o2 = __shfl(orow[2], src_lane), o3 = __shfl(orow[3], src_lane);
            dst = ii == 0 ? o0 : ii == 1 ? o1 : ii == 2 ? o2 : o3;
          }
          if (rt < rows) *reinterpret_cast<uint4*>(out + dst * H + n0 + pc * 8) = v;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  } else {
    float* y = static_cast<float*>(g.out[which]);
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
      if (m < nsub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m * 16 + q * 4 + i;
          if (r < rows) {
            int64_t t;
            float wt;
            if (which == 1) {
              t = row0 + r;
              wt = g.gate[t];
            } else {
              const int f = g.perm[row0 + r];
              t = f / g.k;
              wt = g.row_w[f];
            }
            float* yrow = y + t * g.H + n0 + col;
#pragma unroll
            for (int c = 0; c < 4; ++c) unsafeAtomicAdd(yrow + c * 16, wt * acc[m][c][i]);
          }
        }
      }
    }
  }
}

static inline int gemm_grid(int n_chunks, int S) { return static_cast<int>(8 * S * div_up(n_chunks, 8)); }

static void fill_common(GemmArgs& g, const moe_dims& d, const GemmTiles& tl, int T, bool shared) {
  g.perm = tl.perm;
  g.offsets = tl.offsets;
  g.block_map = tl.block_map;
  g.n_tiles = tl.n_tiles;
  g.block_m = tl.block_m;
  g.n_sh = shared ? tl.n_shared_chunks : 0;
  g.max_tiles = tl.max_tiles;
  g.T = T;
  g.k = d.top_k;
  g.H = d.hidden;
}

hipError_t launch_gemm_swiglu(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* x,
                              const GemmTiles& tl, int T, uint16_t* h, uint16_t* h_sh, hipStream_t s) {
  GemmArgs g{};
  g.codes[0] = w.codes;
  g.scales[0] = w.scales;
  g.biases[0] = w.biases;
  g.K[0] = d.hidden;
  g.N[0] = 2 * d.inter;
  g.Ih[0] = d.inter;
  g.a[0] = x;
  g.lda[0] = d.hidden;
  g.out[0] = h;
  g.ldo[0] = d.inter;
  if (w_sh) {
    g.codes[1] = w_sh->codes;
    g.scales[1] = w_sh->scales;
    g.biases[1] = w_sh->biases;
    g.K[1] = d.hidden;
    g.N[1] = 2 * d.shared_inter;
    g.Ih[1] = d.shared_inter;
    g.a[1] = x;
    g.lda[1] = d.hidden;
    g.out[1] = h_sh;
    g.ldo[1] = d.shared_inter;
  }
  fill_common(g, d, tl, T, w_sh != nullptr);
  const int wmax = w_sh ? max(d.inter, d.shared_inter) : d.inter;
  g.n_slices = static_cast<int>(div_up(wmax, 128));
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<kSwiglu>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

static GemmArgs down_args(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                          const uint16_t* h_sh, const GemmTiles& tl, const float* row_w, const float* gate, int T,
                          void* out) {
  GemmArgs g{};
  g.codes[0] = w.codes;
  g.scales[0] = w.scales;
  g.biases[0] = w.biases;
  g.K[0] = d.inter;
  g.N[0] = d.hidden;
  g.a[0] = h;
  g.lda[0] = d.inter;
  g.out[0] = out;
  g.ldo[0] = d.hidden;
  if (w_sh) {
    g.codes[1] = w_sh->codes;
    g.scales[1] = w_sh->scales;
    g.biases[1] = w_sh->biases;
    g.K[1] = d.shared_inter;
    g.N[1] = d.hidden;
    g.a[1] = h_sh;
    g.lda[1] = d.shared_inter;
    g.out[1] = out;
    g.ldo[1] = d.hidden;
  }
  fill_common(g, d, tl, T, w_sh != nullptr);
  g.row_w = row_w;
  g.gate = gate;
  g.n_slices = static_cast<int>(div_up(d.hidden, 256));
  return g;
}

hipError_t launch_gemm_scatter(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                               const uint16_t* h_sh, const GemmTiles& tl, const float* row_w, const float* gate,
                               int T, float* y, hipStream_t s) {
  GemmArgs g = down_args(d, w, w_sh, h, h_sh, tl, row_w, gate, T, y);
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<kScatter>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_slots(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                             const uint16_t* h_sh, const GemmTiles& tl, const float* row_w, const float* gate, int T,
                             uint16_t* slots, hipStream_t s) {
  GemmArgs g = down_args(d, w, w_sh, h, h_sh, tl, row_w, gate, T, slots);
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<kSlots>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

// out[t][n] = bf16( sum_{j=0..k} slot[t][j][n] ), slots fp16, summed in fp32 in
// slot order (shared expert last).  8 columns per thread.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ slots, uint16_t* __restrict__ out,
                                                 int T, int H, int k) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // 8-column group
  const int per_tok = H / 8;
  if (i >= static_cast<int64_t>(T) * per_tok) return;
  const int64_t t = i / per_tok;
  const int c8 = static_cast<int>(i % per_tok) * 8;
  const uint16_t* src = slots + t * (k + 1) * H + c8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j <= k; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * H);
    const f16x2 p[4] = {__builtin_bit_cast(f16x2, v.x), __builtin_bit_cast(f16x2, v.y),
                        __builtin_bit_cast(f16x2, v.z), __builtin_bit_cast(f16x2, v.w)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[2 * u] += static_cast<float>(p[u].x);
      acc[2 * u + 1] += static_cast<float>(p[u].y);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + t * H + c8) = o;
}

hipError_t launch_combine(const uint16_t* slots, uint16_t* out, int T, int H, int k, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(T) * (H / 8);
  hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>(div_up(n, 256))), dim3(256), 0, s, slots, out, T, H, k);
  return hipGetLastError();
}

}  // namespace moe
