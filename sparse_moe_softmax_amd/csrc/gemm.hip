// Grouped expert GEMMs with int4 weights dequantised in registers.  The
// method expands the quantised weights inside the grouped GEMM, a tile per
// step, so the expanded values exist only in registers and are never written back
// (Inside Lily page, section "Performance Gains and Workload Patterns"); prefill
// is matrix-matrix work for the matrix units (Lily page, section "Why Apple
// Silicon isn't just a smaller datacenter GPU").
//
// Work unit (workgroup of 4 waves) = one tile of up to kBM rows of one expert
// x one slice of 256 weight rows (product columns).  Tiles come from the block
// map (routed experts) and, in the fused layer, from kBM-row chunks of the
// shared expert, which are placed first (the largest tiles start first).
//
// Weights are read in the packed matrix-core layout (moe_prepack_q4): for each
// (expert, slice, 64-wide K block) one contiguous 9216-byte block holding the
// slice's 256 rows of codes (32 B each, already in LDS order) and their
// (scale, bias) pairs, so that one K block of weights is nine fully used 1 KB
// loads instead of 256 partial rows and 512 scattered 2-byte reads.
//
// Data path per 64-wide K block ("stage"), all asynchronous:
//   * global -> LDS direct loads (global_load_lds, no register staging) of
//       - the tile's activation rows, bf16 [rows][64], rows gathered through the
//         permutation; 16-byte chunks XOR-swizzled by row so that MFMA
//         fragment reads are bank-conflict free without padding,
//       - the weight block of the slice (codes, then scale/bias pairs);
//   * a ring of kStages stages in LDS, refilled kStages-1 blocks ahead, with
//     explicit vmcnt waits (every vector-memory instruction inside the loop is
//     one of these loads, issued in a fixed order and count per stage) and one
//     barrier per K block;
//   * each wave reads its 64 columns' codes from LDS and dequantises them in
//     registers into MFMA B fragments: exact fp32 c*s + b, one nearest-even
//     rounding to bf16 (see dequant8), one k-step ahead of the MFMAs that use
//     them.  Dequantised weights never reach LDS or HBM;
//   * v_mfma_f32_32x32x16_bf16 with fp32 accumulators, every A fragment used
//     for both 32-column groups of the wave.
// Two workgroups run on each CU (half the LDS and at most 256 registers per
// lane each), so that one workgroup's start-up latency, epilogue and stalls
// are covered by the other's matrix work; tiles are at most 128 rows.
//
// Epilogues (through LDS so that every lane stores 16 contiguous bytes):
//   SWIGLU : wave columns = 32 gate rows + the matching 32 up rows;
//            h = bf16( silu(gate) * up ) in grouped order.
//   SCATTER: y[token][col] += weight * o, fp32 atomics (standalone op).
//   SLOTS  : the unweighted output o of slot j of a token (routed slots
//            j < k, the shared expert's slot k), token-major [T][k+1][H], as
//            fp16 with a power-of-two exponent per (slot row, 64 columns):
//            slot = fp16(o * 2^-e), e chosen so that the 64-value chunk's
//            largest magnitude lies in [2^14, 2^15): the range is fp32's and
//            every value within 2^28 of its chunk's largest keeps fp16's
//            11-bit precision.  The combine weights and sums them afterwards
//            in a fixed order.  No atomics.
//
// Launch order is XCD-aware: consecutive workgroup ids go round-robin to the 8
// XCDs, so ids are mapped such that all column slices of one tile share an XCD
// (and its L2) and consecutive tiles spread over the XCDs.
#include "internal.hpp"

namespace moe {

constexpr int kGemmThreads = 256;
constexpr int kSliceRows = 256;                  // product columns (weight rows) per slice
constexpr int kBStage = kSliceRows * 32;         // int4 codes of 256 weight rows x 64 K
constexpr int kPackBlock = kBStage + kSliceRows * 4;  // + (fp16 scale, fp16 bias) per row = 9216 B
constexpr int kGemmOcc = 2;                      // workgroups per CU: LDS and registers are split
constexpr int kRingBytes = (160 * 1024 / kGemmOcc - kBM * 12 - 512) / 256 * 256;  // LDS ring shared by all stages
// A stage holds KS consecutive 64-wide K blocks: per block the live rows only
// (MT 32-row sub-tiles, 4 KB each) and the slice's packed weight block.  The
// ring takes as many stages as fit, at most 8 (3 for a 128-row tile).
template <int MT, int KS>
struct Ring {
  static constexpr int kA = MT * 32 * 128;          // activation bytes of one K block
  static constexpr int kStage = KS * (kA + kPackBlock);
  static constexpr int kStages = (kRingBytes / kStage) < 8 ? (kRingBytes / kStage) : 8;
  static_assert(kStages >= 3, "ring too shallow");
};
static_assert(kRingBytes + kBM * 12 <= 160 * 1024 / kGemmOcc, "LDS budget");
static_assert(kRingBytes % 256 == 0, "ring alignment");

enum { kSwiglu = 0, kScatter = 1, kSlots = 2 };

// Slot epilogue staging: a wave's 32 x 64 fp16 sub-tile, rows padded to 144 bytes.
constexpr int kSlotRowBytes = 144;   // 64 fp16 + 16 B pad
constexpr int kSlotStageBytes = 32 * kSlotRowBytes;
static_assert(4 * kSlotStageBytes <= kRingBytes, "slot staging fits the ring");

// Exponent e of a slot chunk whose largest magnitude is mx: mx * 2^-e lies in
// [2^14, 2^15) (for 2^-96 <= mx < 2^128), so every scaled value is finite in
// fp16 (largest finite 65504) and every value within 2^28 of mx is an fp16
// normal with its 11-bit significand.  Integer work on the bits:
// floor(log2(mx)) = biased exponent - 127 for normal mx.  e is kept in
// [-110, 113] so that 2^-e and 2^e are normal floats; stored as int8.
__device__ inline int slot_exponent(float mx) {
  const int fl = static_cast<int>((__float_as_uint(mx) >> 23) & 255u) - 127;
  return min(113, max(-110, fl - 14));
}
// Two floats -> two fp16 (round to nearest even), low half first.
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

struct GemmArgs {
  // index 0: routed experts, 1: shared expert
  const uint8_t* packed[2];   // matrix-core layout
  int64_t expert_bytes[2];    // packed bytes per expert
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
  const int32_t* tile_rows;   // rows per routed tile (NULL: from offsets)
  const float* row_w;   // routed: weight per flat slot (SCATTER)
  const float* gate;    // shared: sigmoid gate per token (SCATTER)
  uint8_t* slot_exp;    // SLOTS: exponent e per (slot row, 64 columns), [T][k+1][H/64]
  int gather;           // routed A rows: 1 = token rows a[perm[p] / k], 0 = a[p]
  int block_m;
  int n_sh;             // shared chunks (first in the chunk order)
  int max_tiles;
  int n_slices;
  int T, k, H;
};

// Stored position of 16-byte half h of weight row i in a B stage (row = 32 B):
// rows are spread so that 8 (or 16) consecutive rows read distinct bank groups.
// Applied once by the packing, so the stage is a plain copy of a packed block.
__host__ __device__ inline int b_half(int i, int h) { return h ^ (((i >> 2) ^ (i >> 3)) & 1); }

// Everything one workgroup needs once its tile and slice are known.
struct Tile {
  int which, row0, rows, K, N, kg, wave, lane, Ih, hc, n0;
  bool active;
  const uint8_t* pbase;   // packed blocks of this expert and slice
};

// K loop + epilogue for a tile of MT 32-row sub-tiles (straight-line code),
// KS K blocks per ring stage.  One-sub-tile tiles (remainder tiles, and every
// tile of a small batch) take two K blocks per stage when the K blocks pair
// up: their iteration is dominated by its fixed chain (wait, barrier, load
// issue, fragment reads), which is then paid once per 128 of K.
//
// MFMA v_mfma_f32_32x32x16_bf16.  Within a K block of 64 the lane group
// g = lane/32 covers K offsets [32g, 32g+32); k-step s (0..3) of a lane holds
// offsets 32g+8s .. 32g+8s+7 for both operands (a consistent permutation of K).
// A fragment: row lane%32 of the sub-tile; B fragment: weight row (column)
// lane%32 of the column group; C: acc[m][c][j] holds row 8(j/4) + 4g + (j%4),
// column lane%32.  The two operand fragments have the same lane layout, so
// swapping them gives the transposed product: the SLOTS epilogue takes it that
// way (acc[m][c][j] then holds row lane%32, column 8(j/4) + 4g + (j%4)), so
// that a lane owns 32 values of one output row.
template <int MODE>
__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (MODE == kSlots)
    return mfma32(b, a, c);
  else
    return mfma32(a, b, c);
}

template <int MODE, int MT, int KS>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const Tile& t, unsigned char* ring,
                                          int64_t* s_drow, float* s_wt) {
  constexpr int kAI = MT;                          // A direct loads per wave per K block (8 rows each)
  constexpr int kDma = KS * (kAI + 3);            // + 2 code loads + scale/bias, per K block
  constexpr int kStages = Ring<MT, KS>::kStages;
  constexpr int kStageBytes = Ring<MT, KS>::kStage;
  constexpr int kAStage = Ring<MT, KS>::kA;        // stage layout: A of each K block, then B of each
  constexpr int kBOff = KS * kAStage;
  static_assert((kStages - 2) * kDma <= 63, "vmcnt range");
  // Where an iteration issues the next stage's loads: the down GEMMs (8 K
  // blocks a tile) issue them right after the first MFMAs of the iteration,
  // so the matrix core starts sooner after the barrier; the gate/up GEMM
  // issues them right after the barrier (it measured slower the other way).
  constexpr bool kLateIssue = MODE != kSwiglu;
  const int wave = t.wave, lane = t.lane;
  const int col = lane & 31, gq = lane >> 5;

  // ---- per-lane sources of the direct loads.  Row indices of a gathered tile
  //      are loaded together first (one wait), then turned into addresses.
  const uint16_t* abase = g.a[t.which];
  const int lda = g.lda[t.which];
  int arow_idx[kAI];
#pragma unroll
  for (int j = 0; j < kAI; ++j) {
    const int r = (wave * kAI + j) * 8 + (lane >> 3);   // tile row this lane fills
    arow_idx[j] = t.row0 + min(r, t.rows - 1);         // padding rows re-read the last live row
  }
  if (g.gather && t.which == 0) {
    int pr[kAI];
#pragma unroll
    for (int j = 0; j < kAI; ++j) pr[j] = g.perm[arow_idx[j]];
#pragma unroll
    for (int j = 0; j < kAI; ++j) arow_idx[j] = pr[j] / g.k;
  }
  uint32_t asrc[kAI];   // byte offsets from abase (a tensor of at most 2^32 bytes)
#pragma unroll
  for (int j = 0; j < kAI; ++j) {
    const int r = (wave * kAI + j) * 8 + (lane >> 3);
    const int p = lane & 7;                            // physical chunk this lane fills
    int c = 0;                                         // logical chunk with a_chunk(r, c) == p
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      if (a_chunk(r, cc) == p) c = cc;
    asrc[j] = (static_cast<uint32_t>(arow_idx[j]) * static_cast<uint32_t>(lda) + c * 8) * 2;
  }
  const i32x4 arsrc = buffer_rsrc(abase);
  // weights: 2 x 1 KB of codes and 256 B of scale/bias pairs per wave and stage
  const i32x4 brsrc = buffer_rsrc(t.pbase);
  const uint32_t bsrc = wave * 2048 + lane * 16;
  const uint32_t ssrc = kBStage + wave * 256 + lane * 4;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave index in a scalar register
  const uint32_t ring_s = lds_addr(ring);

  auto issue = [&](int kb) {
    const uint32_t st = ring_s + (kb % kStages) * kStageBytes;
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const uint32_t aoff = (kb * KS + u) * 128, boff = (kb * KS + u) * kPackBlock;
      const uint32_t sa = st + u * kAStage, sb = st + kBOff + u * kPackBlock;
#pragma unroll
      for (int j = 0; j < kAI; ++j) bdma16(arsrc, asrc[j], aoff, sa + (wave_s * kAI + j) * 1024);
#pragma unroll
      for (int j = 0; j < 2; ++j) bdma16(brsrc, bsrc + j * 1024, boff, sb + wave_s * 2048 + j * 1024);
      bdma4(brsrc, ssrc, boff, sb + kBStage + wave_s * 256);
    }
  };

  f32x16 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][c][j] = 0.f;

  const int kg = t.kg / KS;   // ring stages (iterations)

  // Codes and dequantisation constants of this wave's two 32-column groups in a stage.
  struct BRaw {
    uint4 codes[2];
    DqConst dc[2];
  };
  auto read_b = [&](int kb, int u, BRaw& r) {
    const unsigned char* sb0 = ring + (kb % kStages) * kStageBytes + kBOff + u * kPackBlock;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = wave * 64 + c * 32 + col;
      r.codes[c] = *reinterpret_cast<const uint4*>(sb0 + i * 32 + b_half(i, gq) * 16);
      const uint32_t sb = *reinterpret_cast<const uint32_t*>(sb0 + kBStage + i * 4);
      r.dc[c] = dq_const(static_cast<uint16_t>(sb), static_cast<uint16_t>(sb >> 16));
    }
  };
  // k-step ks of column group c: codes dword ks -> 8 bf16
  auto dq = [&](const BRaw& r, int c, int ks) -> bf16x8 {
    const uint32_t q = ks == 0 ? r.codes[c].x : ks == 1 ? r.codes[c].y : ks == 2 ? r.codes[c].z : r.codes[c].w;
    return __builtin_bit_cast(bf16x8, dequant8(q, r.dc[c].s24, r.dc[c].s20, r.dc[c].bias));
  };
  auto read_a = [&](const unsigned char* st, int ks, bf16x8 (&af)[MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = m * 32 + col;
      af[m] = *reinterpret_cast<const bf16x8*>(st + r * 128 + (a_chunk(r, 4 * gq + ks) << 4));
    }
  };

  // Every wave computes, also an idle one (narrow shared expert, or N not a
  // multiple of the slice) on its dummy rows, whose results are never stored:
  // a branch here would make the compiler shuttle the accumulators between
  // register files on every K block.
  bf16x8 af[2][MT];
  using Steady = std::integral_constant<bool, true>;
  using Drain = std::integral_constant<bool, false>;

  // One K block.  Two workgroups share a CU, so the other workgroup's wave on
  // the same SIMD covers this one's stalls, and an iteration works on its own
  // stage only: it waits for this wave's loads of stage kb (kStages - 2 later
  // stages may stay in flight), barriers (stage kb landed for every wave;
  // stage kb-1 fully consumed), refills the slot of stage kb-1 with stage
  // kb + kStages - 1, reads the stage's codes, and runs the MFMAs with the
  // dequantisation of each k-step's weights (2 column groups) one k-step ahead
  // of the MFMAs that use them and the A fragments also read one k-step ahead;
  // scheduling fences keep that interleaving.
  // STEADY (kb + kStages - 1 < kg): the iteration always issues a stage and
  // waits for a fixed count (one basic block).
  auto iteration = [&](auto steady_tag, int kb) {
    constexpr bool kSteady = decltype(steady_tag)::value;
    if (kSteady)
      wait_vmcnt<(kStages - 2) * kDma>();
    else
      wait_stages<kDma, kStages - 2>(min(kStages - 2, kg - 1 - kb));
    __builtin_amdgcn_s_barrier();   // stage kb landed for every wave; stage kb-1 consumed
    const bool do_issue = kSteady || kb + kStages - 1 < kg;
    if (!kLateIssue && do_issue) issue(kb + kStages - 1);
    const unsigned char* st = ring + (kb % kStages) * kStageBytes;
    BRaw raw[KS];
#pragma unroll
    for (int u = 0; u < KS; ++u) read_b(kb, u, raw[u]);
    read_a(st, 0, af[0]);
    bf16x8 bq[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) bq[0][c] = dq(raw[0], c, 0);
    // k-step q of the stage: K block q / 4, k-step q % 4 within it
    // Each SIMD holds one wave of each of the CU's two workgroups, and a wave
    // does not issue its own VALU work while its own MFMA runs: the matrix
    // core is kept busy by the other wave's MFMAs.  In the gate/up GEMM the
    // wave in its MFMA section issues ahead of the other wave's set-up work
    // (barrier, load issue, fragment reads); the down GEMM's short K loops
    // lose by it, so there the priority stays even.
    if constexpr (MODE == kSwiglu) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < 4 * KS; ++q) {
      const int nu = (q + 1) >> 2, nks = (q + 1) & 3;
      if (q + 1 < 4 * KS) read_a(st + nu * kAStage, nks, af[(q + 1) & 1]);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][c] = mma<MODE>(af[q & 1][m], bq[q & 1][c], acc[m][c]);
        if (kLateIssue && q == 0 && c == 0 && do_issue) issue(kb + kStages - 1);
        if (q + 1 < 4 * KS) bq[(q + 1) & 1][c] = dq(raw[nu], c, nks);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (MODE == kSwiglu) __builtin_amdgcn_s_setprio(0);
  };

  // Short tiles (1-2 sub-tiles) have registers to spare, and their iteration
  // is mostly fixed latency: there an iteration dequantises the NEXT stage's
  // weights while the MFMAs use the current stage's (dequantised one
  // iteration earlier), and waits for stage kb+1 instead of kb.
  auto iteration_ahead = [&](auto steady_tag, int kb, bf16x8 (&bcur)[2][4], bf16x8 (&bnext)[2][4]) {
    constexpr bool kSteady = decltype(steady_tag)::value;
    const bool more = kSteady || kb + 1 < kg;
    // issued so far: stages 0 .. min(kb + kStages - 2, kg - 1); wait for stage kb+1
    if (kSteady)
      wait_vmcnt<(kStages - 3) * kDma>();
    else if (more)
      wait_stages<kDma, kStages - 3>(min(kStages - 3, kg - 2 - kb));
    BRaw raw;
    if (more) read_b(kb + 1, 0, raw);   // this wave's own loads: no barrier needed
    __builtin_amdgcn_s_barrier();    // stage kb+1 landed for every wave; stage kb-1 consumed
    const bool do_issue = kSteady || kb + kStages - 1 < kg;
    if (!kLateIssue && do_issue) issue(kb + kStages - 1);
    const unsigned char* st = ring + (kb % kStages) * kStageBytes;
    const unsigned char* st_next = ring + ((kb + 1) % kStages) * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3)
        read_a(st, ks + 1, af[(ks + 1) & 1]);
      else if (more)
        read_a(st_next, 0, af[0]);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][c] = mma<MODE>(af[ks & 1][m], bcur[c][ks], acc[m][c]);
        if (kLateIssue && ks == 0 && c == 0 && do_issue) issue(kb + kStages - 1);
        if (more) bnext[c][ks] = dq(raw, c, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // prologue: stages 0 .. kStages-2 in flight
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < kg) issue(s);
  // slots: this thread's row's flat slot, needed only at the epilogue
  constexpr bool deferred_rows = MODE == kSlots;
  int my_f = 0;
  if (deferred_rows && t.which == 0 && static_cast<int>(threadIdx.x) < t.rows) my_f = g.perm[t.row0 + threadIdx.x];
  const int steady_end = kg - (kStages - 1);   // iterations kb < steady_end are steady
  if constexpr (MT <= 2 && KS == 1) {
    static_assert(Ring<MT, KS>::kStages >= 3, "the ahead loop waits one stage ahead");
    // stage 0 landed, dequantised, and its first A fragments read
    wait_stages<kDma, kStages - 2>(min(kStages - 2, kg - 1));
    __builtin_amdgcn_s_barrier();
    bf16x8 b0[2][4], b1[2][4];
    {
      BRaw raw;
      read_b(0, 0, raw);
      read_a(ring, 0, af[0]);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b0[c][ks] = dq(raw, c, ks);
    }
    int kb = 0;
    for (; kb + 2 <= steady_end; kb += 2) {
      iteration_ahead(Steady{}, kb, b0, b1);
      iteration_ahead(Steady{}, kb + 1, b1, b0);
    }
    for (; kb + 2 <= kg; kb += 2) {
      iteration_ahead(Drain{}, kb, b0, b1);
      iteration_ahead(Drain{}, kb + 1, b1, b0);
    }
    if (kb < kg) iteration_ahead(Drain{}, kb, b0, b1);
  } else {
    int kb = 0;
    for (; kb < steady_end; ++kb) iteration(Steady{}, kb);
    for (; kb < kg; ++kb) iteration(Drain{}, kb);
  }

  // ---- epilogue.  Each wave stages one 32-row sub-tile at a time in a private
  // 4 KB LDS area at the start of the ring, which is free once every wave has
  // left the loop; stores are then 16 contiguous bytes per lane.
  __syncthreads();
  if (deferred_rows) {
    const int r = threadIdx.x;
    if (r < t.rows) {
      const int k = g.k;
      s_drow[r] = t.which == 1 ? static_cast<int64_t>(t.row0 + r) * (k + 1) + k
                               : static_cast<int64_t>(my_f / k) * (k + 1) + (my_f % k);
    }
    __syncthreads();
  }
  if (!t.active) return;
  const int rows = t.rows, row0 = t.row0;
  unsigned char* stg = ring + wave * 4096;
  if (MODE == kSwiglu) {
    uint16_t* out = static_cast<uint16_t*>(g.out[t.which]);
    const int ldo = g.ldo[t.which];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      // 32 rows x 32 h columns, bf16 (64 B per row)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float gt = acc[m][0][j];
        const float up = acc[m][1][j];
        const float h = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
        const int r = (j >> 2) * 8 + gq * 4 + (j & 3);
        reinterpret_cast<uint16_t*>(stg)[r * 32 + col] = f32_to_bf16_bits(h);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        // lane -> row 16 part + lane/4, 16-byte piece lane%4
        const int r = part * 16 + (lane >> 2), pc = lane & 3;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 64 + pc * 16);
        const int rt = m * 32 + r;
        if (rt < rows) *reinterpret_cast<uint4*>(out + static_cast<int64_t>(row0 + rt) * ldo + t.hc + pc * 8) = v;
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else if (MODE == kSlots) {
    // The products are transposed here (see mma): a lane owns 32 values of
    // row `col` of the sub-tile, the 4-column runs 8i + 4g .. 8i + 4g + 3 of
    // the wave's 64 columns.  The row's largest magnitude is the lane's own
    // maximum combined with that of lane ^ 32 (the other runs).  The values
    // scaled by 2^-e go to fp16 and are staged as rows of 64 fp16 (+16 B pad)
    // so that stores are 16 contiguous bytes per lane; lane g == 0 stores the
    // row's exponent byte.
    uint16_t* out = static_cast<uint16_t*>(g.out[0]);   // [T][k+1][H] fp16
    const int H = g.H;
    const int chunk = t.n0 >> 6, n_chunks = H >> 6;
    unsigned char* st16 = ring + wave * kSlotStageBytes;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float mx = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(acc[m][c][j]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const int e = slot_exponent(mx);
      const float sc = __int_as_float((127 - e) << 23);   // 2^-e, exact scaling
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 v = {pack_f16x2(acc[m][c][4 * i] * sc, acc[m][c][4 * i + 1] * sc),
                           pack_f16x2(acc[m][c][4 * i + 2] * sc, acc[m][c][4 * i + 3] * sc)};
          *reinterpret_cast<uint2*>(st16 + col * kSlotRowBytes + (c * 32 + 8 * i + 4 * gq) * 2) = v;
        }
      if (gq == 0 && m * 32 + col < rows)
        g.slot_exp[s_drow[m * 32 + col] * n_chunks + chunk] = static_cast<uint8_t>(e & 255);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        const int r = part * 8 + (lane >> 3), pc = lane & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(st16 + r * kSlotRowBytes + pc * 16);
        if (m * 32 + r < rows)
          *reinterpret_cast<uint4*>(out + s_drow[m * 32 + r] * H + t.n0 + pc * 8) = v;
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    float* y = static_cast<float*>(g.out[t.which]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = m * 32 + (j >> 2) * 8 + gq * 4 + (j & 3);
        if (r < rows) {
          float* yrow = y + s_drow[r] * g.H + t.n0 + col;
          const float wt = s_wt[r];
#pragma unroll
          for (int c = 0; c < 2; ++c) unsafeAtomicAdd(yrow + c * 32, wt * acc[m][c][j]);
        }
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, kGemmOcc) void k_gemm_q4(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRingBytes];

  // ---- which tile / slice
  const int wg = blockIdx.x;
  const int S = g.n_slices;
  const int xcd = wg & 7;
  const int rr = wg >> 3;
  const int chunk = (rr / S) * 8 + xcd;
  const int slice = rr % S;
  if (chunk >= g.n_sh + g.max_tiles) return;
  Tile t;
  int e;
  if (chunk < g.n_sh) {
    t.which = 1;
    e = 0;
    t.row0 = chunk * kBM;
    t.rows = min(kBM, g.T - t.row0);
  } else {
    const int tile = chunk - g.n_sh;
    if (tile >= *g.n_tiles) return;
    t.which = 0;
    e = g.block_map[2 * tile];
    t.row0 = g.block_map[2 * tile + 1];
    // the tile's height arrives with its block-map entry when the grouping
    // wrote it, else it follows from the expert's segment end
    t.rows = g.tile_rows ? g.tile_rows[tile] : min(g.block_m, g.offsets[e + 1] - t.row0);
  }
  t.K = g.K[t.which];
  t.N = g.N[t.which];
  t.kg = t.K / 64;
  const int tid = threadIdx.x;
  t.lane = tid & 63;
  t.wave = tid >> 6;
  t.Ih = 0;
  t.hc = 0;
  t.n0 = 0;
  if (MODE == kSwiglu) {
    t.Ih = g.Ih[t.which];
    if (slice * 128 >= t.Ih) return;  // whole block idle (narrower shared expert)
    t.hc = slice * 128 + t.wave * 32;
    t.active = t.hc < t.Ih;
  } else {
    t.n0 = slice * 256 + t.wave * 64;
    t.active = t.n0 < t.N;
  }
  t.pbase = g.packed[t.which] + static_cast<int64_t>(e) * g.expert_bytes[t.which] +
            static_cast<int64_t>(slice) * t.kg * kPackBlock;

  // Output row and weight of every tile row (down projection epilogues).  The
  // scatter epilogue fills them before the K loop, whose first barrier
  // publishes them.  Slots need only the output row: gemm_tile loads the
  // permutation after issuing its first stages and fills s_drow at the
  // epilogue, so that load adds no latency to the start.
  __shared__ int64_t s_drow[kBM];
  __shared__ float s_wt[kBM];
  if (MODE == kScatter) {
    for (int r = tid; r < t.rows; r += kGemmThreads) {
      const int k = g.k;
      if (t.which == 1) {
        const int tok = t.row0 + r;
        s_drow[r] = tok;
        s_wt[r] = g.gate ? g.gate[tok] : 1.0f;
      } else {
        const int f = g.perm[t.row0 + r];
        s_drow[r] = f / k;
        s_wt[r] = g.row_w[f];
      }
    }
  }

  switch ((t.rows + 31) >> 5) {
#define MOE_MT_CASE(n) \
  case n:              \
    gemm_tile<MODE, n, 1>(g, t, ring, s_drow, s_wt); \
    break;
    case 1:
      if ((t.kg & 1) == 0)
        gemm_tile<MODE, 1, 2>(g, t, ring, s_drow, s_wt);
      else
        gemm_tile<MODE, 1, 1>(g, t, ring, s_drow, s_wt);
      break;
    MOE_MT_CASE(2) MOE_MT_CASE(3)
#if MOE_BM > 96
    MOE_MT_CASE(4)
#endif
#if MOE_BM > 128
    MOE_MT_CASE(5) MOE_MT_CASE(6)
#endif
#if MOE_BM > 192
    MOE_MT_CASE(7) MOE_MT_CASE(8)
#endif
#undef MOE_MT_CASE
    default:
      break;
  }
}

static inline int gemm_grid(int n_chunks, int S) { return static_cast<int>(8 * S * div_up(n_chunks, 8)); }

static void fill_common(GemmArgs& g, const moe_dims& d, const GemmTiles& tl, int T, bool shared) {
  g.perm = tl.perm;
  g.offsets = tl.offsets;
  g.block_map = tl.block_map;
  g.n_tiles = tl.n_tiles;
  g.tile_rows = tl.tile_rows;
  g.block_m = tl.block_m;
  g.n_sh = shared ? tl.n_shared_chunks : 0;
  g.max_tiles = tl.max_tiles;
  g.T = T;
  g.k = d.top_k;
  g.H = d.hidden;
}

hipError_t launch_gemm_swiglu(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* x,
                              bool gather, const GemmTiles& tl, int T, uint16_t* h, uint16_t* h_sh, hipStream_t s) {
  GemmArgs g{};
  g.packed[0] = w.packed;
  g.expert_bytes[0] = pack_geom(d, MOE_MAT_GATE_UP).expert_bytes;
  g.K[0] = d.hidden;
  g.N[0] = 2 * d.inter;
  g.Ih[0] = d.inter;
  g.a[0] = x;
  g.lda[0] = d.hidden;
  g.out[0] = h;
  g.ldo[0] = d.inter;
  if (w_sh) {
    g.packed[1] = w_sh->packed;
    g.expert_bytes[1] = pack_geom(d, MOE_MAT_SH_GATE_UP).expert_bytes;
    g.K[1] = d.hidden;
    g.N[1] = 2 * d.shared_inter;
    g.Ih[1] = d.shared_inter;
    g.a[1] = x;
    g.lda[1] = d.hidden;
    g.out[1] = h_sh;
    g.ldo[1] = d.shared_inter;
  }
  fill_common(g, d, tl, T, w_sh != nullptr);
  g.gather = gather ? 1 : 0;
  const int wmax = w_sh ? max(d.inter, d.shared_inter) : d.inter;
  g.n_slices = static_cast<int>(div_up(wmax, 128));
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<kSwiglu>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

static GemmArgs down_args(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h, bool gather,
                          const uint16_t* h_sh, const GemmTiles& tl, const float* row_w, const float* gate, int T,
                          void* out) {
  GemmArgs g{};
  g.packed[0] = w.packed;
  g.expert_bytes[0] = pack_geom(d, MOE_MAT_DOWN).expert_bytes;
  g.K[0] = d.inter;
  g.N[0] = d.hidden;
  g.a[0] = h;
  g.lda[0] = d.inter;
  g.out[0] = out;
  g.ldo[0] = d.hidden;
  if (w_sh) {
    g.packed[1] = w_sh->packed;
    g.expert_bytes[1] = pack_geom(d, MOE_MAT_SH_DOWN).expert_bytes;
    g.K[1] = d.shared_inter;
    g.N[1] = d.hidden;
    g.a[1] = h_sh;
    g.lda[1] = d.shared_inter;
    g.out[1] = out;
    g.ldo[1] = d.hidden;
  }
  fill_common(g, d, tl, T, w_sh != nullptr);
  g.gather = gather ? 1 : 0;
  g.row_w = row_w;
  g.gate = gate;
  g.n_slices = static_cast<int>(div_up(d.hidden, 256));
  return g;
}

hipError_t launch_gemm_scatter(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                               bool gather, const uint16_t* h_sh, const GemmTiles& tl, const float* row_w,
                               const float* gate, int T, float* y, hipStream_t s) {
  GemmArgs g = down_args(d, w, w_sh, h, gather, h_sh, tl, row_w, gate, T, y);
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<kScatter>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_slots(const moe_dims& d, const moe_q4& w, const moe_q4* w_sh, const uint16_t* h,
                             const uint16_t* h_sh, const GemmTiles& tl, int T, uint16_t* slots, uint8_t* slot_exp,
                             hipStream_t s) {
  GemmArgs g = down_args(d, w, w_sh, h, false, h_sh, tl, nullptr, nullptr, T, slots);
  g.slot_exp = slot_exp;
  const int grid = gemm_grid(g.n_sh + g.max_tiles, g.n_slices);
  hipLaunchKernelGGL(k_gemm_q4<kSlots>, dim3(grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

// Canonical -> packed weights: one thread per (expert, slice, K block, packed
// row) copies the row's 32 code bytes of the block into its LDS-order position
// and its (scale, bias) pair.  Rows past the matrix are zero.
__global__ __launch_bounds__(256) void k_prepack_q4(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ biases, uint8_t* __restrict__ packed,
                                                    PackGeom pg) {
  const int i = threadIdx.x;                 // packed row in the slice
  const int64_t blk = blockIdx.x;            // ((e * slices) + s) * kg + kb
  const int kb = static_cast<int>(blk % pg.kg);
  const int sl = static_cast<int>((blk / pg.kg) % pg.slices);
  const int64_t e = blk / (static_cast<int64_t>(pg.kg) * pg.slices);
  int n;
  if (pg.swiglu) {
    const int w = i >> 6, r = i & 63;
    const int hcol = sl * 128 + w * 32 + (r & 31);
    n = hcol < pg.Iw ? ((r < 32) ? hcol : pg.Iw + hcol) : -1;
  } else {
    n = sl * kSliceRows + i;
    n = n < pg.N ? n : -1;
  }
  uint8_t* out = packed + e * pg.expert_bytes + blk % (static_cast<int64_t>(pg.kg) * pg.slices) * kPackBlock;
  uint4 c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
  uint32_t sb = 0;
  if (n >= 0) {
    const uint8_t* src = codes + (e * pg.N + n) * (pg.K / 2) + kb * 32;
    c0 = *reinterpret_cast<const uint4*>(src);
    c1 = *reinterpret_cast<const uint4*>(src + 16);
    const int64_t gi = (e * pg.N + n) * pg.kg + kb;
    sb = static_cast<uint32_t>(scales[gi]) | (static_cast<uint32_t>(biases[gi]) << 16);
  }
  *reinterpret_cast<uint4*>(out + i * 32 + b_half(i, 0) * 16) = c0;
  *reinterpret_cast<uint4*>(out + i * 32 + b_half(i, 1) * 16) = c1;
  *reinterpret_cast<uint32_t*>(out + kBStage + i * 4) = sb;
}

hipError_t launch_prepack_q4(const moe_dims& d, int matrix, const moe_q4& w, int n_exp, uint8_t* packed,
                             hipStream_t s) {
  const PackGeom pg = pack_geom(d, matrix);
  const int64_t blocks = static_cast<int64_t>(n_exp) * pg.slices * pg.kg;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prepack_q4, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, w.codes, w.scales,
                     w.biases, packed, pg);
  return hipGetLastError();
}

// out[t][n] = bf16( sum_{j<k} w[t][j] * o_j + gate[t] * o_k ), o_j = slot[t][j][n] * 2^e[t][j][n/64]
// (fp16 slot values and their chunk exponents as the slot epilogue wrote
// them), summed in fp32 in slot order (shared expert last); w or gate NULL =
// weights of 1.  The weight and 2^e are multiplied first (exact: a power-of-two
// scaling, unless w * 2^e falls below fp32's normal range, which needs chunks
// near 2^-96), so each term is the single rounding of w * o.  8 columns per
// thread.  With k known at compile time (K > 0) all k + 1 slot vectors and
// exponents are requested before the sum, so a thread waits for one memory
// round trip, not k + 1; K = 0 takes k at run time.
template <int K>
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ slots,
                                                 const uint8_t* __restrict__ slot_exp, const float* __restrict__ w,
                                                 const float* __restrict__ gate, uint16_t* __restrict__ out, int T,
                                                 int H, int k_rt) {
  const int k = K > 0 ? K : k_rt;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // 8-column group
  const int per_tok = H / 8;
  if (i >= static_cast<int64_t>(T) * per_tok) return;
  const int64_t t = i / per_tok;
  const int c8 = static_cast<int>(i % per_tok) * 8;
  const int n_chunks = H >> 6;
  const uint16_t* src = slots + t * (k + 1) * H + c8;
  const uint8_t* esrc = slot_exp + t * (k + 1) * n_chunks + (c8 >> 6);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4& v, float wj, int e) {
    const float we = wj * __int_as_float((127 + e) << 23);   // w * 2^e
    const f16x2 p[4] = {__builtin_bit_cast(f16x2, v.x), __builtin_bit_cast(f16x2, v.y),
                        __builtin_bit_cast(f16x2, v.z), __builtin_bit_cast(f16x2, v.w)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[2 * u] = __builtin_fmaf(we, static_cast<float>(p[u].x), acc[2 * u]);
      acc[2 * u + 1] = __builtin_fmaf(we, static_cast<float>(p[u].y), acc[2 * u + 1]);
    }
  };
  if constexpr (K > 0) {
    uint4 v[K + 1];
    int e[K + 1];
#pragma unroll
    for (int j = 0; j <= K; ++j) {
      v[j] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * H);
      e[j] = static_cast<int8_t>(esrc[j * n_chunks]);
    }
    float wj[K + 1];
#pragma unroll
    for (int j = 0; j < K; ++j) wj[j] = w ? w[t * K + j] : 1.0f;
    wj[K] = gate ? gate[t] : 1.0f;
#pragma unroll
    for (int j = 0; j <= K; ++j) add(v[j], wj[j], e[j]);
  } else {
    for (int j = 0; j <= k; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * H);
      add(v, j == k ? (gate ? gate[t] : 1.0f) : (w ? w[t * k + j] : 1.0f), static_cast<int8_t>(esrc[j * n_chunks]));
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + t * H + c8) = o;
}

hipError_t launch_combine(const uint16_t* slots, const uint8_t* slot_exp, const float* w, const float* gate,
                          uint16_t* out, int T, int H, int k, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(T) * (H / 8);
  const dim3 grid(static_cast<unsigned>(div_up(n, 256)));
  if (k == 8)
    hipLaunchKernelGGL(k_combine<8>, grid, dim3(256), 0, s, slots, slot_exp, w, gate, out, T, H, k);
  else
    hipLaunchKernelGGL(k_combine<0>, grid, dim3(256), 0, s, slots, slot_exp, w, gate, out, T, H, k);
  return hipGetLastError();
}

}  // namespace moe
