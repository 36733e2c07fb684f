// Runs every entry point of the CPU oracle on small random inputs, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py:
// any out-of-bounds access, use after free, signed overflow or misaligned
// access in the oracle ends the run with a report.  Also checks a few
// invariants so that the calls are known to have done their work.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int oracle_abi_version(void);
void oracle_round_bf16(const double* in, double* out, int64_t n);
void oracle_bf16_bits(const double* in, uint16_t* out, int64_t n);
void oracle_half_to_double(const uint16_t* in, double* out, int64_t n);
void oracle_bf16_to_double(const uint16_t* in, double* out, int64_t n);
void oracle_dequant(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N, int64_t K,
                    int64_t G, double* out);
void oracle_router(const uint16_t* x, int64_t T, int64_t H, int64_t E, const float* W, const float* bias,
                   const float* wsg, float* logits, float* s, int n_threads);
void oracle_topk(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids, float* w);
void oracle_sigmoid(const float* s, int64_t T, float* g);
int oracle_group(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t BM, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv_perm, int32_t* block_map, int64_t max_tiles, int32_t* n_tiles);
void oracle_grouped_swiglu(int64_t H, int64_t I, int64_t E, int64_t G, int64_t k, const uint16_t* a,
                           int rows_are_tokens, const int32_t* perm, const int32_t* offsets, const uint8_t* codes,
                           const uint16_t* scales, const uint16_t* biases, uint16_t* h_out, int n_threads);
void oracle_grouped_down(int64_t H, int64_t I, int64_t E, int64_t G, const uint16_t* h, const int32_t* offsets,
                         const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, double* o_out,
                         int n_threads);
void oracle_moe_tokens(int64_t H, int64_t I, int64_t E, int64_t k, int64_t G, int64_t Is, const uint16_t* x,
                       const int32_t* ids, const float* w, const float* g, const uint8_t* gu_codes,
                       const uint16_t* gu_scales, const uint16_t* gu_biases, const uint8_t* dn_codes,
                       const uint16_t* dn_scales, const uint16_t* dn_biases, const uint8_t* sgu_codes,
                       const uint16_t* sgu_scales, const uint16_t* sgu_biases, const uint8_t* sdn_codes,
                       const uint16_t* sdn_scales, const uint16_t* sdn_biases, const int32_t* tokens, int64_t n_tok,
                       uint16_t* out, double* y_out, uint16_t* h_out, uint16_t* h_sh_out, int n_threads);
void oracle_gqa_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* lens, int64_t B,
                       int64_t Hq, int64_t Hkv, int64_t S, int64_t D, double scale, double* out, int n_threads);
}

#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(1);                                            \
    }                                                          \
  } while (0)

static std::mt19937_64 rng(12345);
static uint16_t bf16_of(float f) {  // truncation is enough for test inputs
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}

struct Q4 {
  std::vector<uint8_t> c;
  std::vector<uint16_t> s, b;
};
static Q4 q4(int64_t n_exp, int64_t N, int64_t K, int64_t G) {
  Q4 q;
  q.c.resize(n_exp * N * K / 2);
  q.s.resize(n_exp * N * (K / G));
  q.b.resize(q.s.size());
  for (auto& v : q.c) v = static_cast<uint8_t>(rng());
  for (size_t i = 0; i < q.s.size(); ++i) {
    q.s[i] = static_cast<uint16_t>(0x2000 + rng() % 0x0800);  // fp16 scales around 0.008-0.016
    q.b[i] = static_cast<uint16_t>(q.s[i] | 0x8000) + 0x0C00;  // a negative bias of similar size
  }
  return q;
}

int main() {
  CHECK(oracle_abi_version() == 1);
  const int64_t H = 128, I = 64, E = 16, k = 4, G = 64, Is = 192, T = 37;
  // scalars
  std::vector<double> d(1000), r(1000);
  std::vector<uint16_t> bits(1000);
  for (auto& v : d) v = std::ldexp(static_cast<double>(rng() % 100000) - 50000.0, -10);
  oracle_round_bf16(d.data(), r.data(), 1000);
  oracle_bf16_bits(d.data(), bits.data(), 1000);
  oracle_bf16_to_double(bits.data(), d.data(), 1000);
  for (int i = 0; i < 1000; ++i) CHECK(d[i] == r[i]);
  std::vector<uint16_t> all(65536);
  std::vector<double> dd(65536);
  for (int i = 0; i < 65536; ++i) all[i] = static_cast<uint16_t>(i);
  oracle_half_to_double(all.data(), dd.data(), 65536);
  oracle_bf16_to_double(all.data(), dd.data(), 65536);
  // weights and inputs
  Q4 gu = q4(E, 2 * I, H, G), dn = q4(E, H, I, G), sgu = q4(1, 2 * Is, H, G), sdn = q4(1, H, Is, G);
  std::vector<double> deq(2 * I * H);
  oracle_dequant(gu.c.data(), gu.s.data(), gu.b.data(), 2 * I, H, G, deq.data());
  std::vector<uint16_t> x(T * H);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (auto& v : x) v = bf16_of(nd(rng));
  std::vector<float> W(E * H), wsg(H), bias(E), logits(T * E), s(T), gt(T), w(T * k);
  for (auto& v : W) v = nd(rng) * 0.05f;
  for (auto& v : wsg) v = nd(rng) * 0.05f;
  for (auto& v : bias) v = nd(rng);
  for (int threads : {1, 3}) oracle_router(x.data(), T, H, E, W.data(), bias.data(), wsg.data(), logits.data(),
                                           s.data(), threads);
  std::vector<int32_t> ids(T * k);
  oracle_topk(logits.data(), T, E, k, ids.data(), w.data());
  oracle_sigmoid(s.data(), T, gt.data());
  for (int64_t t = 0; t < T; ++t) {
    double sum = 0;
    for (int64_t j = 0; j < k; ++j) sum += w[t * k + j];
    CHECK(std::fabs(sum - 1.0) < 1e-5);
  }
  // grouping, also with a block map that is too small
  const int64_t BM = 5, max_tiles = (T * k + BM - 1) / BM + E;
  std::vector<int32_t> counts(E), offsets(E + 1), perm(T * k), inv(T * k), bmap(2 * max_tiles), nt(1);
  CHECK(oracle_group(ids.data(), T, k, E, BM, counts.data(), offsets.data(), perm.data(), inv.data(), bmap.data(),
                     max_tiles, nt.data()) == 0);
  CHECK(offsets[E] == T * k);
  CHECK(oracle_group(ids.data(), T, k, E, BM, counts.data(), offsets.data(), perm.data(), inv.data(), bmap.data(), 1,
                     nt.data()) != 0);
  // experts
  std::vector<uint16_t> h(T * k * I), hs(T * I);
  for (int threads : {1, 4})
    oracle_grouped_swiglu(H, I, E, G, k, x.data(), 1, perm.data(), offsets.data(), gu.c.data(), gu.s.data(),
                          gu.b.data(), h.data(), threads);
  std::vector<double> o(T * k * H);
  oracle_grouped_down(H, I, E, G, h.data(), offsets.data(), dn.c.data(), dn.s.data(), dn.b.data(), o.data(), 2);
  std::vector<int32_t> tok(T);
  for (int64_t t = 0; t < T; ++t) tok[t] = static_cast<int32_t>(T - 1 - t);
  std::vector<uint16_t> out(T * H), hh(T * k * I), hsh(T * Is);
  std::vector<double> y(T * H);
  for (int threads : {1, 5})
    oracle_moe_tokens(H, I, E, k, G, Is, x.data(), ids.data(), w.data(), gt.data(), gu.c.data(), gu.s.data(),
                      gu.b.data(), dn.c.data(), dn.s.data(), dn.b.data(), sgu.c.data(), sgu.s.data(), sgu.b.data(),
                      sdn.c.data(), sdn.s.data(), sdn.b.data(), tok.data(), T, out.data(), y.data(), hh.data(),
                      hsh.data(), threads);
  // attention
  const int64_t B = 2, Hq = 4, Hkv = 2, S = 9, D = 64;
  std::vector<uint16_t> q(B * Hq * D), kc(B * Hkv * S * D), vc(kc.size());
  for (auto& v : q) v = bf16_of(nd(rng));
  for (auto& v : kc) v = bf16_of(nd(rng));
  for (auto& v : vc) v = bf16_of(nd(rng));
  std::vector<int32_t> lens = {0, 7};
  std::vector<double> ao(B * Hq * D);
  oracle_gqa_decode(q.data(), kc.data(), vc.data(), lens.data(), B, Hq, Hkv, S, D, 0.125, ao.data(), 2);
  for (int64_t i = 0; i < Hq * D; ++i) CHECK(ao[i] == 0.0);   // empty sequence
  std::printf("oracle driver: ok\n");
  return 0;
}
