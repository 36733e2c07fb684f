// Plain, slow CPU oracle for the sparse Mixture-of-Experts layer.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
// this file; only the test-suite, the smoke check and the benchmark's CPU
// baseline do.  It shares no code, header, table or helper with the HIP library.
//
// What it computes (the pages: "Lily: Perplexity's Custom Inference Engine for
// Apple Silicon", section "The architecture that forces the issue: MoE plus
// Gated DeltaNet" -- each token is scored against 256 experts, keeps the best
// eight, and also passes through one shared expert; "Inside Lily ...", section "Performance
// Gains and Workload Patterns" -- 4-bit weights rebuilt tile by tile inside the
// grouped GEMM, routing histograms and block maps kept on the GPU).  The pages
// give no formulas; the precise definition used here (softmax over the router
// logits, top-k on the logit with ties to the lower expert index, renormalised
// weights, SwiGLU experts, affine int4 groups of 64 along the input dimension,
// sigmoid-gated shared expert) is the plainest reading and is written out step
// by step below.
//
// Precision contract:
//   * every dot product is accumulated in double, in ascending index order;
//   * a dequantised weight is fp32(c)*fp32(scale) + fp32(bias) rounded to fp32,
//     then rounded once (nearest-even) to bfloat16;
//   * the SwiGLU output h is rounded once (nearest-even) to bfloat16 from the
//     double value; the layer output likewise;
//   * router logits are the double dot product rounded to fp32 (plus an fp32
//     bias add when a per-expert bias is given); routing weights and the
//     shared gate are evaluated in double and stored as fp32.
//
// Built with g++ -O2 -ffp-contract=off (no fast-math).  Threads only split
// independent tokens or experts; they never change an arithmetic order.
//
// Also here: one decode step of grouped-query attention (oracle_gqa_decode),
// the attention the same model runs in its full-attention layers (Lily page,
// section "The architecture that forces the issue": 16 query heads share 2
// key/value heads) and whose packed form the "Inside Lily ..." page lists
// among its optimisations (section "Key Optimizations at a Glance", GQA
// packing).  The pages give no formula; the reading is the standard one
// written out below: query head h reads key/value head h / (Hq / Hkv), scores
// are scale * (q . k_p) over the L cached positions of its sequence, softmax
// over those positions, output the softmax-weighted sum of the value rows, in
// double, rounded once to bfloat16 by the caller's comparison.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- numbers

// IEEE binary16 bit pattern -> exact double.
double half_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int ex = (h >> 10) & 31;
  const int man = h & 1023;
  double v;
  if (ex == 0) {
    v = std::ldexp(static_cast<double>(man), -24);            // subnormal
  } else if (ex == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(man + 1024), ex - 25);  // (1 + m/1024) 2^(ex-15)
  }
  return sign ? -v : v;
}

// bfloat16 bit pattern -> exact double (1 sign, 8 exponent, 7 mantissa bits).
double bf16_to_double(uint16_t b) {
  const int sign = b >> 15;
  const int ex = (b >> 7) & 255;
  const int man = b & 127;
  double v;
  if (ex == 0) {
    v = std::ldexp(static_cast<double>(man), -133);            // subnormal
  } else if (ex == 255) {
    v = man ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(man + 128), ex - 134);  // (1 + m/128) 2^(ex-127)
  }
  return sign ? -v : v;
}

const double kBf16Max = std::ldexp(255.0, 120);  // (2 - 2^-7) * 2^127

// Round a double to the nearest bfloat16 value, ties to even, in one step.
double round_bf16(double v) {
  if (v == 0.0 || !std::isfinite(v)) return v;
  const double a = std::fabs(v);
  int e = 0;
  std::frexp(a, &e);              // a = m * 2^e with m in [0.5, 1): leading bit 2^(e-1)
  int q = e - 8;                  // 8 significant bits -> spacing 2^(e-8)
  if (q < -133) q = -133;         // below 2^-126 the spacing stays 2^-133
  // a * 2^-q < 2^8, so the scaled value and its rounding are exact in double;
  // nearbyint uses the default rounding mode, round-to-nearest-even.
  double r = std::ldexp(std::nearbyint(std::ldexp(a, -q)), q);
  if (r > kBf16Max) r = INFINITY;
  return std::copysign(r, v);
}

// bfloat16 bit pattern of a value that is already a bfloat16 number.
uint16_t bf16_bits(double v) {
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0;
  if (std::isinf(v)) return v < 0 ? 0xFF80 : 0x7F80;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  int e = 0;
  const double m = std::frexp(a, &e);  // a = m 2^e
  int biased = e - 1 + 127;            // exponent field of a normal number
  if (biased <= 0) {                   // subnormal: a = man * 2^-133
    return sign | static_cast<uint16_t>(std::ldexp(a, 133));
  }
  const int man = static_cast<int>(std::ldexp(m, 8)) - 128;  // 8-bit significand minus hidden bit
  return sign | static_cast<uint16_t>(biased << 7) | static_cast<uint16_t>(man);
}

// Dequantised weight: v = fp32(c)*fp32(s) + fp32(b) rounded to fp32, then to bf16.
double dequant_one(int code, uint16_t scale_h, uint16_t bias_h) {
  const double s = half_to_double(scale_h);
  const double b = half_to_double(bias_h);
  const float v = static_cast<float>(static_cast<double>(code) * s + b);
  return round_bf16(static_cast<double>(v));
}

// A matrix of one expert in the affine int4 format: codes [N][K/2] (element
// (n, k) in byte k/2, low nibble = even k), fp16 scale and bias [N][K/G].
struct Q4 {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
};

Q4 expert_slice(const Q4& all, int64_t e, int64_t N, int64_t K, int64_t G) {
  Q4 q;
  q.codes = all.codes + e * N * (K / 2);
  q.scales = all.scales + e * N * (K / G);
  q.biases = all.biases + e * N * (K / G);
  return q;
}

// Dense dequantised matrix [N][K] of one expert, values exactly bf16.
std::vector<double> dequant_matrix(const Q4& q, int64_t N, int64_t K, int64_t G) {
  std::vector<double> w(static_cast<size_t>(N * K));
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = q.codes[n * (K / 2) + k / 2];
      const int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
      const int64_t g = n * (K / G) + k / G;
      w[n * K + k] = dequant_one(code, q.scales[g], q.biases[g]);
    }
  }
  return w;
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// One expert on one activation row a[K=H]:
//   gate_n = sum_k a_k W[n][k], up_n = sum_k a_k W[I+n][k]   (double, k ascending)
//   h_n    = bf16( silu(gate_n) * up_n )
void expert_swiglu_row(const double* a, const double* wgu, int64_t H, int64_t I, double* h) {
  for (int64_t n = 0; n < I; ++n) {
    const double* wg = wgu + n * H;
    const double* wu = wgu + (I + n) * H;
    double gate = 0.0, up = 0.0;
    for (int64_t k = 0; k < H; ++k) gate += a[k] * wg[k];
    for (int64_t k = 0; k < H; ++k) up += a[k] * wu[k];
    h[n] = round_bf16(silu(gate) * up);
  }
}

// o_m = sum_n h_n Wd[m][n]   (double, n ascending), Wd is [H][I].
void expert_down_row(const double* h, const double* wd, int64_t H, int64_t I, double* o) {
  for (int64_t m = 0; m < H; ++m) {
    const double* w = wd + m * I;
    double acc = 0.0;
    for (int64_t n = 0; n < I; ++n) acc += h[n] * w[n];
    o[m] = acc;
  }
}

int pick_threads(int n_threads, int64_t work) {
  int t = n_threads > 0 ? n_threads : static_cast<int>(std::thread::hardware_concurrency());
  if (t < 1) t = 1;
  if (work < t) t = static_cast<int>(std::max<int64_t>(work, 1));
  return t;
}

// Run f(i) for i in [0, n) on up to n_threads threads (dynamic hand-out).
template <class F>
void parallel_for(int64_t n, int n_threads, F f) {
  const int t = pick_threads(n_threads, n);
  if (t == 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int64_t> next(0);
  std::vector<std::thread> pool;
  for (int w = 0; w < t; ++w) {
    pool.emplace_back([&]() {
      for (;;) {
        const int64_t i = next.fetch_add(1);
        if (i >= n) break;
        f(i);
      }
    });
  }
  for (auto& th : pool) th.join();
}

// Dequantised matrices of the experts in `need`, computed once each.
struct ExpertCache {
  std::vector<std::vector<double>> gu, dn;
};

void fill_cache(ExpertCache& c, const std::vector<int64_t>& need, const Q4& gu_all, const Q4& dn_all,
                int64_t H, int64_t I, int64_t G, int n_threads) {
  parallel_for(static_cast<int64_t>(need.size()), n_threads, [&](int64_t i) {
    const int64_t e = need[i];
    c.gu[e] = dequant_matrix(expert_slice(gu_all, e, 2 * I, H, G), 2 * I, H, G);
    c.dn[e] = dequant_matrix(expert_slice(dn_all, e, H, I, G), H, I, G);
  });
}

}  // namespace

extern "C" {

int oracle_abi_version(void) { return 1; }

// ---------------------------------------------------------------- scalars (pinned by tests)

void oracle_round_bf16(const double* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(in[i]);
}

void oracle_bf16_bits(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits(round_bf16(in[i]));
}

void oracle_half_to_double(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = half_to_double(in[i]);
}

void oracle_bf16_to_double(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_double(in[i]);
}

// Dequantise one [N][K] matrix; out holds the bf16 values as doubles.
void oracle_dequant(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                    int64_t K, int64_t G, double* out) {
  Q4 q{codes, scales, biases};
  std::vector<double> w = dequant_matrix(q, N, K, G);
  std::memcpy(out, w.data(), w.size() * sizeof(double));
}

// ---------------------------------------------------------------- router

// logits[t][e] = fp32( sum_k x[t][k] W[e][k] ) (+ bias[e] in fp32 when bias != null)
// s[t]         = fp32( sum_k x[t][k] wsg[k] )
void oracle_router(const uint16_t* x, int64_t T, int64_t H, int64_t E, const float* W, const float* bias,
                   const float* wsg, float* logits, float* s, int n_threads) {
  parallel_for(T, n_threads, [&](int64_t t) {
    std::vector<double> a(static_cast<size_t>(H));
    for (int64_t k = 0; k < H; ++k) a[k] = bf16_to_double(x[t * H + k]);
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t k = 0; k < H; ++k) acc += a[k] * static_cast<double>(W[e * H + k]);
      float l = static_cast<float>(acc);
      if (bias) l = l + bias[e];
      logits[t * E + e] = l;
    }
    if (wsg && s) {
      double acc = 0.0;
      for (int64_t k = 0; k < H; ++k) acc += a[k] * static_cast<double>(wsg[k]);
      s[t] = static_cast<float>(acc);
    }
  });
}

// ---------------------------------------------------------------- top-k routing

// Softmax over all E logits, keep the k experts with the largest logits (ties
// to the lower expert index; the slot order is that ranking), renormalise the
// kept probabilities so they sum to one.
void oracle_topk(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids, float* w) {
  std::vector<int32_t> order(static_cast<size_t>(E));
  std::vector<double> p(static_cast<size_t>(E));
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    double mx = -INFINITY;
    for (int64_t e = 0; e < E; ++e) mx = std::max(mx, static_cast<double>(l[e]));
    double den = 0.0;
    for (int64_t e = 0; e < E; ++e) {
      p[e] = std::exp(static_cast<double>(l[e]) - mx);
      den += p[e];
    }
    for (int64_t e = 0; e < E; ++e) p[e] /= den;
    for (int64_t e = 0; e < E; ++e) order[e] = static_cast<int32_t>(e);
    // Descending logit; stable sort keeps the ascending expert index among equal logits.
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return l[a] > l[b]; });
    double kept = 0.0;
    for (int64_t j = 0; j < k; ++j) kept += p[order[j]];
    for (int64_t j = 0; j < k; ++j) {
      ids[t * k + j] = order[j];
      w[t * k + j] = static_cast<float>(p[order[j]] / kept);
    }
  }
}

// Shared-expert gate g = 1 / (1 + exp(-s)).
void oracle_sigmoid(const float* s, int64_t T, float* g) {
  for (int64_t t = 0; t < T; ++t) g[t] = static_cast<float>(1.0 / (1.0 + std::exp(-static_cast<double>(s[t]))));
}

// ---------------------------------------------------------------- grouping

// counts[e]  : number of flat slots f = t*k + j routed to expert e
// offsets    : exclusive prefix sum of counts, offsets[E] = T*k
// perm[p]    : the flat slots sorted by expert, ascending flat index within an expert
// inv_perm[f]: position of slot f in perm
// block_map  : for e ascending, m ascending: (e, offsets[e] + m*BM) for each of the
//              ceil(counts[e]/BM) tiles; entries past n_tiles are (-1, -1)
// Returns 0, or -1 if max_tiles is too small.
int oracle_group(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t BM, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* block_map, int64_t max_tiles,
                 int32_t* n_tiles) {
  const int64_t F = T * k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < F; ++f) counts[ids[f]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(static_cast<size_t>(E), 0);
  for (int64_t f = 0; f < F; ++f) {
    const int32_t e = ids[f];
    const int32_t p = offsets[e] + fill[e]++;
    perm[p] = static_cast<int32_t>(f);
    inv_perm[f] = p;
  }
  int64_t nt = 0;
  for (int64_t e = 0; e < E; ++e) {
    for (int64_t m = 0; m * BM < counts[e]; ++m) {
      if (nt >= max_tiles) return -1;
      block_map[2 * nt] = static_cast<int32_t>(e);
      block_map[2 * nt + 1] = static_cast<int32_t>(offsets[e] + m * BM);
      ++nt;
    }
  }
  for (int64_t i = nt; i < max_tiles; ++i) {
    block_map[2 * i] = -1;
    block_map[2 * i + 1] = -1;
  }
  *n_tiles = static_cast<int32_t>(nt);
  return 0;
}

// ---------------------------------------------------------------- experts, grouped form

// h[p] = SwiGLU of activation row a[row(p)] through expert e(p), for every
// position p of the grouped order: rows come from perm (row = perm[p] / k)
// when rows_are_tokens != 0, else row = p.  Output: h as bf16 bit patterns
// [n_rows][I].  Experts are processed one after another (segment by segment).
void oracle_grouped_swiglu(int64_t H, int64_t I, int64_t E, int64_t G, int64_t k, const uint16_t* a,
                           int rows_are_tokens, const int32_t* perm, const int32_t* offsets,
                           const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                           uint16_t* h_out, int n_threads) {
  const Q4 all{codes, scales, biases};
  parallel_for(E, n_threads, [&](int64_t e) {
    const int64_t lo = offsets[e], hi = offsets[e + 1];
    if (hi <= lo) return;
    const std::vector<double> w = dequant_matrix(expert_slice(all, e, 2 * I, H, G), 2 * I, H, G);
    std::vector<double> row(static_cast<size_t>(H)), h(static_cast<size_t>(I));
    for (int64_t p = lo; p < hi; ++p) {
      const int64_t r = rows_are_tokens ? perm[p] / k : p;
      for (int64_t q = 0; q < H; ++q) row[q] = bf16_to_double(a[r * H + q]);
      expert_swiglu_row(row.data(), w.data(), H, I, h.data());
      for (int64_t n = 0; n < I; ++n) h_out[p * I + n] = bf16_bits(h[n]);
    }
  });
}

// o[p] = h[p] . Wd[e(p)]^T as doubles [n_rows][H], grouped order.
void oracle_grouped_down(int64_t H, int64_t I, int64_t E, int64_t G, const uint16_t* h, const int32_t* offsets,
                         const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, double* o_out,
                         int n_threads) {
  const Q4 all{codes, scales, biases};
  parallel_for(E, n_threads, [&](int64_t e) {
    const int64_t lo = offsets[e], hi = offsets[e + 1];
    if (hi <= lo) return;
    const std::vector<double> w = dequant_matrix(expert_slice(all, e, H, I, G), H, I, G);
    std::vector<double> hr(static_cast<size_t>(I));
    for (int64_t p = lo; p < hi; ++p) {
      for (int64_t n = 0; n < I; ++n) hr[n] = bf16_to_double(h[p * I + n]);
      expert_down_row(hr.data(), w.data(), H, I, o_out + p * H);
    }
  });
}

// ---------------------------------------------------------------- the layer, token by token

// For each listed token t (tokens[i]):
//   y = sum_j w[t][j] * Expert_{ids[t][j]}(x[t])  (j ascending)  +  g[t] * Shared(x[t])
//   out[i] = bf16(y)   (bit patterns [n_tok][H]); y_out[i] = y (doubles, may be null)
// h_out (nullable) receives the routed h rows [n_tok][k][I] and h_sh_out
// (nullable) the shared h rows [n_tok][Is], both as bf16 bit patterns.
void oracle_moe_tokens(int64_t H, int64_t I, int64_t E, int64_t k, int64_t G, int64_t Is, const uint16_t* x,
                       const int32_t* ids, const float* w, const float* g, const uint8_t* gu_codes,
                       const uint16_t* gu_scales, const uint16_t* gu_biases, const uint8_t* dn_codes,
                       const uint16_t* dn_scales, const uint16_t* dn_biases, const uint8_t* sgu_codes,
                       const uint16_t* sgu_scales, const uint16_t* sgu_biases, const uint8_t* sdn_codes,
                       const uint16_t* sdn_scales, const uint16_t* sdn_biases, const int32_t* tokens,
                       int64_t n_tok, uint16_t* out, double* y_out, uint16_t* h_out, uint16_t* h_sh_out,
                       int n_threads) {
  const Q4 gu_all{gu_codes, gu_scales, gu_biases};
  const Q4 dn_all{dn_codes, dn_scales, dn_biases};
  // Dequantise each expert the listed tokens touch, once.
  std::vector<char> used(static_cast<size_t>(E), 0);
  for (int64_t i = 0; i < n_tok; ++i)
    for (int64_t j = 0; j < k; ++j) used[ids[tokens[i] * k + j]] = 1;
  std::vector<int64_t> need;
  for (int64_t e = 0; e < E; ++e)
    if (used[e]) need.push_back(e);
  ExpertCache cache;
  cache.gu.resize(static_cast<size_t>(E));
  cache.dn.resize(static_cast<size_t>(E));
  fill_cache(cache, need, gu_all, dn_all, H, I, G, n_threads);
  const std::vector<double> sgu =
      dequant_matrix(Q4{sgu_codes, sgu_scales, sgu_biases}, 2 * Is, H, G);
  const std::vector<double> sdn = dequant_matrix(Q4{sdn_codes, sdn_scales, sdn_biases}, H, Is, G);

  parallel_for(n_tok, n_threads, [&](int64_t i) {
    const int64_t t = tokens[i];
    std::vector<double> a(static_cast<size_t>(H)), y(static_cast<size_t>(H), 0.0);
    std::vector<double> h(static_cast<size_t>(std::max(I, Is))), o(static_cast<size_t>(H));
    for (int64_t q = 0; q < H; ++q) a[q] = bf16_to_double(x[t * H + q]);
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = ids[t * k + j];
      expert_swiglu_row(a.data(), cache.gu[e].data(), H, I, h.data());
      if (h_out)
        for (int64_t n = 0; n < I; ++n) h_out[(i * k + j) * I + n] = bf16_bits(h[n]);
      expert_down_row(h.data(), cache.dn[e].data(), H, I, o.data());
      const double wj = static_cast<double>(w[t * k + j]);
      for (int64_t m = 0; m < H; ++m) y[m] += wj * o[m];
    }
    expert_swiglu_row(a.data(), sgu.data(), H, Is, h.data());
    if (h_sh_out)
      for (int64_t n = 0; n < Is; ++n) h_sh_out[i * Is + n] = bf16_bits(h[n]);
    expert_down_row(h.data(), sdn.data(), H, Is, o.data());
    const double gt = static_cast<double>(g[t]);
    for (int64_t m = 0; m < H; ++m) y[m] += gt * o[m];
    for (int64_t m = 0; m < H; ++m) {
      out[i * H + m] = bf16_bits(round_bf16(y[m]));
      if (y_out) y_out[i * H + m] = y[m];
    }
  });
}


// One decode step of grouped-query attention for B sequences.
//   q   [B][Hq][D] bf16 bits, k/v [B][Hkv][S][D] bf16 bits (S cached positions
//   per sequence and head), lens[B] positions in use (0 <= lens[b] <= S).
//   out [B][Hq][D] double: for query head h of sequence b, with kv = h / (Hq/Hkv),
//   s_p = scale * sum_d q[d] k[p][d]  (p < lens[b]),
//   out = sum_p exp(s_p - max s) v[p] / sum_p exp(s_p - max s);
//   a sequence with no positions gives zeros.
void oracle_gqa_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* lens, int64_t B,
                       int64_t Hq, int64_t Hkv, int64_t S, int64_t D, double scale, double* out, int n_threads) {
  const int64_t group = Hq / Hkv;
  parallel_for(B * Hq, n_threads, [&](int64_t bh) {
    const int64_t b = bh / Hq, h = bh % Hq, kv = h / group;
    const int64_t L = lens[b];
    double* o = out + bh * D;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (L <= 0) return;
    const uint16_t* qh = q + bh * D;
    const uint16_t* kh = kc + (b * Hkv + kv) * S * D;
    const uint16_t* vh = vc + (b * Hkv + kv) * S * D;
    std::vector<double> sc(L);
    double m = -INFINITY;
    for (int64_t p = 0; p < L; ++p) {
      double dot = 0.0;
      for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qh[d]) * bf16_to_double(kh[p * D + d]);
      sc[p] = scale * dot;
      m = std::max(m, sc[p]);
    }
    double den = 0.0;
    for (int64_t p = 0; p < L; ++p) {
      sc[p] = std::exp(sc[p] - m);
      den += sc[p];
    }
    for (int64_t p = 0; p < L; ++p)
      for (int64_t d = 0; d < D; ++d) o[d] += sc[p] * bf16_to_double(vh[p * D + d]);
    for (int64_t d = 0; d < D; ++d) o[d] /= den;
  });
}

}  // extern "C"
