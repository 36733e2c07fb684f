// Grouped expert GEMMs with int4 weights dequantised in registers
// ("By reconstructing 4-bit weights one tile at a time within grouped GEMM
// operations, Lily keeps the expanded arrays inside GPU registers": Inside
// Lily page, section "Performance Gains and Workload Patterns"; prefill work
// is matrix-matrix and belongs on the matrix units: Lily page, section "Why
// Apple Silicon isn't just a smaller datacenter GPU").
//
// Work unit (workgroup) = one tile of up to kBM rows of one expert x one slice
// of weight columns.  Tiles come from the block map (routed experts) and, in
// the fused layer, from kBM-row chunks of the shared expert placed first.
//
//   * A (activation rows, bf16): gathered rows staged per 64-wide K block in
//     LDS, double-buffered, read as MFMA A fragments by all four waves.
//   * B (weights): every wave owns 64 weight rows (columns of the product);
//     each lane loads 8 bytes of int4 codes per column group and K block from
//     global memory, dequantises them in registers into two bf16 MFMA B
//     fragments (exact fp32 c*s+b, one nearest-even rounding to bf16), and
//     reuses them across all row sub-tiles of the tile.  Dequantised weights
//     never touch LDS or HBM.
//   * MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulators for kBM rows x 64
//     columns per wave.  Inside a K block of 64 the lane group q = lane/16
//     covers K offsets [16q, 16q+16) and fragment s holds 16q+8s .. +7 for both
//     operands -- a consistent permutation of K (the sum is unchanged), chosen
//     so a lane's codes are 8 contiguous bytes and its A data 32 contiguous bytes.
//
// Epilogues:
//   SWIGLU : wave columns are 32 gate rows + the matching 32 up rows;
//            h = bf16( silu(gate) * up ) stored in grouped order.
//   SCATTER: y[token][col] += weight * o with fp32 atomics (routed: weight =
//            routing weight of the slot; shared: the sigmoid gate).
//
// Launch order is XCD-aware: consecutive workgroup ids go round-robin to the 8
// XCDs, so ids are mapped such that all column slices of one tile share an XCD
// (and its L2) and consecutive tiles spread over the XCDs.
#include "internal.hpp"

namespace moe {

constexpr int kLdA = 64 + 8;  // padded LDS row of the A tile (144 B)
constexpr int kGemmThreads = 256;

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
  const float* row_w;   // SCATTER routed: weight per flat slot
  const float* gate;    // SCATTER shared: sigmoid gate per token
  int block_m;
  int n_sh;             // shared chunks (first in the chunk order)
  int max_tiles;
  int n_slices;
  int T, k, H;
};

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_q4(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdA];

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

  // ---- this wave's 64 weight rows (4 column groups of 16)
  int wrow[4];
  bool active;
  if (MODE == 0) {
    const int Ih = g.Ih[which];
    const int hc = slice * 128 + wave * 32;
    if (slice * 128 >= Ih) return;  // whole block idle (narrower shared expert)
    active = hc < Ih;
    wrow[0] = hc + col;
    wrow[1] = hc + 16 + col;
    wrow[2] = Ih + hc + col;
    wrow[3] = Ih + hc + 16 + col;
  } else {
    const int n0 = slice * 256 + wave * 64;
    active = n0 < N;
    for (int c = 0; c < 4; ++c) wrow[c] = n0 + c * 16 + col;
  }
  if (!active)
    for (int c = 0; c < 4; ++c) wrow[c] = 0;
  const int kg = K / 64;  // quantisation groups (= K blocks) per row
  const uint8_t* cbase = g.codes[which] + static_cast<int64_t>(e) * N * (K / 2);
  const uint16_t* sbase = g.scales[which] + static_cast<int64_t>(e) * N * kg;
  const uint16_t* bbase = g.biases[which] + static_cast<int64_t>(e) * N * kg;

  // ---- A staging: thread handles 16-byte chunk c8 of rows r_i = tid/8 + 32 i
  const int c8 = tid & 7;
  const uint16_t* asrc[kBM / 32];
#pragma unroll
  for (int i = 0; i < kBM / 32; ++i) {
    const int r = (tid >> 3) + 32 * i;
    asrc[i] = nullptr;
    if (r < rows) {
      int64_t arow;
      if (which == 1)
        arow = row0 + r;
      else if (MODE == 0)
        arow = g.perm[row0 + r] / g.k;
      else
        arow = row0 + r;
      asrc[i] = g.a[which] + arow * g.lda[which] + c8 * 8;
    }
  }

  uint4 areg[kBM / 32];
  uint2 bcur[4], bnext[4];
  uint16_t scur[4], snext[4], zcur[4], znext[4];

  auto load_a = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kBM / 32; ++i)
      areg[i] = asrc[i] ? *reinterpret_cast<const uint4*>(asrc[i] + kb * 64) : make_uint4(0, 0, 0, 0);
  };
  auto load_b = [&](int kb, uint2 (&b)[4], uint16_t (&s)[4], uint16_t (&z)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      b[c] = *reinterpret_cast<const uint2*>(cbase + static_cast<int64_t>(wrow[c]) * (K / 2) + kb * 32 + q * 8);
      s[c] = sbase[static_cast<int64_t>(wrow[c]) * kg + kb];
      z[c] = bbase[static_cast<int64_t>(wrow[c]) * kg + kb];
    }
  };

  f32x4 acc[kMSub][4];
#pragma unroll
  for (int m = 0; m < kMSub; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsub = (rows + 15) >> 4;
  load_a(0);
  load_b(0, bcur, scur, zcur);

  for (int kb = 0; kb < kg; ++kb) {
    uint16_t* Ab = As[kb & 1];
#pragma unroll
    for (int i = 0; i < kBM / 32; ++i)
      *reinterpret_cast<uint4*>(Ab + ((tid >> 3) + 32 * i) * kLdA + c8 * 8) = areg[i];
    __syncthreads();
    if (kb + 1 < kg) {
      load_a(kb + 1);
      load_b(kb + 1, bnext, snext, znext);
    }
    if (active) {
      bf16x8 bf[4][2];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const DqConst dc = dq_const(scur[c], zcur[c]);
        const uint4 lo = dequant8(bcur[c].x, dc.s24, dc.s20, dc.bias);
        const uint4 hi = dequant8(bcur[c].y, dc.s24, dc.s20, dc.bias);
        bf[c][0] = __builtin_bit_cast(bf16x8, lo);
        bf[c][1] = __builtin_bit_cast(bf16x8, hi);
      }
#pragma unroll
      for (int m = 0; m < kMSub; ++m) {
        if (m < nsub) {
          const uint16_t* ap = Ab + (m * 16 + col) * kLdA + q * 16;
          const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ap);
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ap + 8);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[m][c] = mfma16(a0, bf[c][0], acc[m][c]);
            acc[m][c] = mfma16(a1, bf[c][1], acc[m][c]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bcur[c] = bnext[c];
      scur[c] = snext[c];
      zcur[c] = znext[c];
    }
  }
  if (!active) return;

  // ---- epilogue.  C fragment: lane holds rows 4q..4q+3 of a 16-row sub-tile, column `col`.
  if (MODE == 0) {
    uint16_t* out = static_cast<uint16_t*>(g.out[which]);
    const int ldo = g.ldo[which];
    const int hc = slice * 128 + wave * 32;
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
      if (m < nsub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m * 16 + q * 4 + i;
          if (r < rows) {
            uint16_t* orow = out + static_cast<int64_t>(row0 + r) * ldo + hc;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float gt = acc[m][c][i];
              const float up = acc[m][c + 2][i];
              const float h = gt / (1.0f + __expf(-gt)) * up;
              orow[c * 16 + col] = f32_to_bf16_bits(h);
            }
          }
        }
      }
    }
  } else {
    float* y = static_cast<float*>(g.out[which]);
    const int n0 = slice * 256 + wave * 64;
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
  g.perm = tl.perm;
  g.offsets = tl.offsets;
  g.block_map = tl.block_map;
  g.n_tiles = tl.n_tiles;
  g.block_m = tl.block_m;
  g.n_sh = w_sh ? tl.n_shared_chunks : 0;
  g.max_tiles = tl.max_tiles;
  const int wmax = w_sh ? max(d.inter, d.shared_inter) : d.inter;
  g.n_slices = static_cast<int>(div_up(wmax, 128));
  g.T = T;
  g.k = d.top_k;
  g.H = d.hidden;
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<0>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_scatter(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                               const uint16_t* h_sh, const GemmTiles& tl, const float* row_w, const float* gate,
                               int T, float* y, hipStream_t s) {
  GemmArgs g{};
  g.codes[0] = w.codes;
  g.scales[0] = w.scales;
  g.biases[0] = w.biases;
  g.K[0] = d.inter;
  g.N[0] = d.hidden;
  g.a[0] = h;
  g.lda[0] = d.inter;
  g.out[0] = y;
  g.ldo[0] = d.hidden;
  if (w_sh) {
    g.codes[1] = w_sh->codes;
    g.scales[1] = w_sh->scales;
    g.biases[1] = w_sh->biases;
    g.K[1] = d.shared_inter;
    g.N[1] = d.hidden;
    g.a[1] = h_sh;
    g.lda[1] = d.shared_inter;
    g.out[1] = y;
    g.ldo[1] = d.hidden;
  }
  g.perm = tl.perm;
  g.offsets = tl.offsets;
  g.block_map = tl.block_map;
  g.n_tiles = tl.n_tiles;
  g.row_w = row_w;
  g.gate = gate;
  g.block_m = tl.block_m;
  g.n_sh = w_sh ? tl.n_shared_chunks : 0;
  g.max_tiles = tl.max_tiles;
  g.n_slices = static_cast<int>(div_up(d.hidden, 256));
  g.T = T;
  g.k = d.top_k;
  g.H = d.hidden;
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<1>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

// y (fp32) -> out (bf16, nearest-even), 8 values per thread.
__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ y, uint16_t* __restrict__ out,
                                                  int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(y)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(y)[2 * i + 1];
  uint4 o;
  o.x = pack_bf16x2(a.x, a.y);
  o.y = pack_bf16x2(a.z, a.w);
  o.z = pack_bf16x2(b.x, b.y);
  o.w = pack_bf16x2(b.z, b.w);
  reinterpret_cast<uint4*>(out)[i] = o;
}

hipError_t launch_finalize(const float* y, uint16_t* out, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_finalize, dim3(static_cast<unsigned>(div_up(n8, 256))), dim3(256), 0, s, y, out, n8);
  return hipGetLastError();
}

}  // namespace moe
