// Drives every entry point of the CPU oracle (oracle/vsel_oracle.cpp) once per
// case, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.  The
// cases are small seeded rows with the edge cases the oracle handles: NaN and
// +inf rows, -inf masks, all -inf rows, ties, one-element rows, k = vocab,
// every filter of the sampler chain and of the filtered speculative rules,
// temperature 0, fail-closed sequences.  The outputs are not checked here
// (the Python pins do that); the sanitizers report any invalid access or
// undefined operation and end the run with a nonzero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

extern "C" {
void oracle_chunk_geometry(int64_t n, int64_t chunk, int64_t* count, int64_t* tail);
int oracle_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, uint32_t* out_idx,
                  float* out_val, int nthreads);
int oracle_argmax_excluding(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                            const uint32_t* excluded, int64_t n_excluded, uint32_t* out_idx, uint32_t* out_status,
                            int nthreads);
int oracle_lse(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, double temperature,
               double* out_lse, int nthreads);
int oracle_topk(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k, float* out_vals,
                uint32_t* out_ids, uint32_t* out_argmax, double* out_lse, int nthreads);
int oracle_sample(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, float temperature,
                  int32_t top_k, float top_p, const float* u, uint32_t* out_token, double* out_logp, double* margins,
                  int nthreads);
int oracle_sample_chain(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, float temperature,
                        float top_n_sigma, int32_t top_k, float typical_p, float top_p, float min_p, const float* u,
                        uint32_t* out_token, double* out_logp, double* margins, int nthreads);
int oracle_spec_accept(const float* target, int64_t ld_t, const float* draft, int64_t ld_d, int64_t batch,
                       int32_t gamma, int64_t vocab, float temperature, int32_t top_k, float top_p, float min_p,
                       const uint32_t* draft_tokens, const float* u_acc, const float* u_res, const float* u_bon,
                       int32_t* len_mrs, uint32_t* tok_mrs, int32_t* len_aa, uint32_t* tok_aa, double* summin,
                       double* acc_margin, double* draw_margin, double* filter_margin, int nthreads);
int oracle_spec_match(const float* target, int64_t ld_t, const float* draft, int64_t ld_d, int64_t batch,
                      int32_t gamma, int64_t vocab, float temperature, int32_t top_k, float top_p, float min_p,
                      const uint32_t* draft_tokens, const float* u_match, int32_t* len_sm, uint32_t* tok_sm,
                      double* sumprod, double* match_margin, double* filter_margin, int nthreads);
}

namespace {

constexpr float kNegInf = -std::numeric_limits<float>::infinity();
int failures = 0;

void expect_ok(int rc, const char* what) {
  if (rc != 0) {
    std::fprintf(stderr, "oracle rejected %s\n", what);
    ++failures;
  }
}

// rows x ld float32 with special rows: 0 normal, 1 NaN, 2 +inf, 3 all -inf,
// 4 a third -inf, 5 ties on a coarse grid, 6 one finite element; the pad
// [vocab, ld) holds NaN.
std::vector<float> make_rows(int64_t rows, int64_t vocab, int64_t ld, uint32_t seed) {
  std::mt19937 g(seed);
  std::normal_distribution<float> nd(0.0f, 2.0f);
  std::vector<float> x((size_t)(rows * ld), std::numeric_limits<float>::quiet_NaN());
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < vocab; ++i) {
      float v = nd(g);
      switch (r % 7) {
        case 1: if (i == vocab / 2) v = std::numeric_limits<float>::quiet_NaN(); break;
        case 2: if (i == vocab - 1) v = std::numeric_limits<float>::infinity(); break;
        case 3: v = kNegInf; break;
        case 4: if (i % 3 == 0) v = kNegInf; break;
        case 5: v = std::round(v * 2.0f) / 2.0f; break;
        case 6: v = (i == vocab / 3) ? 0.5f : kNegInf; break;
        default: break;
      }
      x[(size_t)(r * ld + i)] = v;
    }
  return x;
}

std::vector<float> uniforms(int64_t n, uint32_t seed) {
  std::mt19937 g(seed);
  std::uniform_real_distribution<float> ud(0.0f, 1.0f);
  std::vector<float> u((size_t)n);
  for (auto& v : u) v = ud(g);
  return u;
}

void selection(int64_t rows, int64_t vocab, int64_t ld, int threads) {
  const std::vector<float> x = make_rows(rows, vocab, ld, (uint32_t)(rows * 131 + vocab));
  std::vector<uint16_t> xb(x.size());
  for (size_t i = 0; i < x.size(); ++i) {
    uint32_t b;
    std::memcpy(&b, &x[i], 4);
    xb[i] = (uint16_t)(b >> 16);
  }
  const std::vector<float> u = uniforms(rows, (uint32_t)vocab);
  std::vector<uint32_t> idx((size_t)rows), st((size_t)rows), tok((size_t)rows);
  std::vector<float> val((size_t)rows);
  std::vector<double> lse((size_t)rows), logp((size_t)rows), mg2((size_t)rows * 2), mg6((size_t)rows * 6);
  for (int dt = 0; dt < 2; ++dt) {
    const void* p = dt == 0 ? (const void*)x.data() : (const void*)xb.data();
    expect_ok(oracle_argmax(p, dt, rows, vocab, ld, idx.data(), val.data(), threads), "argmax");
    const uint32_t ex[5] = {0u, (uint32_t)(vocab - 1), (uint32_t)vocab + 7u, 0u, (uint32_t)(vocab / 2)};
    expect_ok(oracle_argmax_excluding(p, dt, rows, vocab, ld, ex, 5, idx.data(), st.data(), threads), "excluding");
    expect_ok(oracle_argmax_excluding(p, dt, rows, vocab, ld, nullptr, 0, idx.data(), st.data(), threads),
              "excluding (empty set)");
    for (double T : {1.0, 0.3}) expect_ok(oracle_lse(p, dt, rows, vocab, ld, T, lse.data(), threads), "lse");
    for (int64_t k : {int64_t(1), std::min<int64_t>(vocab, 5), vocab}) {
      std::vector<float> v((size_t)(rows * k));
      std::vector<uint32_t> ids((size_t)(rows * k)), am((size_t)rows);
      expect_ok(oracle_topk(p, dt, rows, vocab, ld, (int32_t)k, v.data(), ids.data(), am.data(), lse.data(), threads),
                "topk");
    }
    const float Ts[3] = {0.0f, 0.7f, 1.5f};
    for (float T : Ts)
      for (int32_t k : {0, 1, 2, 20})
        for (float tp : {1.0f, 0.9f}) {
          if (k == 0 && tp < 1.0f) continue;
          expect_ok(oracle_sample(p, dt, rows, vocab, ld, T, std::min<int32_t>(k, (int32_t)vocab), tp, u.data(),
                                  tok.data(), logp.data(), mg2.data(), threads),
                    "sample");
        }
    struct Chain { float sig; int32_t k; float typ, tp, mp; };
    const Chain chains[] = {{0, 0, 1, 1, 0}, {1.0f, 0, 1, 1, 0.05f}, {0, 0, 0.9f, 1, 0}, {0, 0, 0.5f, 0.9f, 0.1f},
                            {2.0f, 0, 1, 0.8f, 0}, {1.0f, 50, 0.9f, 0.95f, 0.05f}, {0, 3, 0.3f, 1, 1.0f}};
    for (float T : Ts)
      for (const Chain& c : chains)
        expect_ok(oracle_sample_chain(p, dt, rows, vocab, ld, T, c.sig, std::min<int32_t>(c.k, (int32_t)vocab), c.typ,
                                      c.tp, c.mp, u.data(), tok.data(), logp.data(), mg6.data(), threads),
                  "sample_chain");
  }
}

void speculative(int64_t B, int32_t G, int64_t vocab, int threads) {
  const int64_t nT = B * (G + 1), nD = B * G, ld = vocab + 3;
  std::mt19937 g((uint32_t)(B * 17 + G * 5 + vocab));
  std::normal_distribution<float> nd(0.0f, 2.0f);
  std::vector<float> t((size_t)(nT * ld)), d((size_t)(nD * ld));
  for (auto& v : t) v = nd(g);
  for (auto& v : d) v = nd(g);
  if (B > 2) {
    t[(size_t)(1 * (G + 1) * ld + 2)] = std::numeric_limits<float>::quiet_NaN();  // sequence 1 fails closed
    for (int64_t i = 0; i < vocab; i += 2) d[(size_t)(2 * G * ld + i)] = kNegInf;  // masks in a draft row
  }
  std::vector<uint32_t> toks((size_t)nD);
  for (int64_t i = 0; i < nD; ++i) toks[(size_t)i] = (uint32_t)(g() % (uint32_t)vocab);
  if (B > 3) toks[(size_t)(3 * G)] = (uint32_t)vocab;  // an out-of-range draft
  const std::vector<float> ua = uniforms(nD, 1), ur = uniforms(nD, 2), ub = uniforms(B, 3), um = uniforms(nT, 4);
  std::vector<int32_t> lm((size_t)B), la((size_t)B), ls((size_t)B);
  std::vector<uint32_t> tm((size_t)nT), ta((size_t)nT), tsm((size_t)nT);
  std::vector<double> smin((size_t)nD), sprod((size_t)nD), am((size_t)nD), dm((size_t)B), fm((size_t)B),
      mm((size_t)nT), fm2((size_t)B);
  struct Filt { int32_t k; float tp, mp; };
  const Filt filts[] = {{0, 1, 0}, {5, 1, 0}, {0, 0.9f, 0}, {0, 1, 0.05f}, {7, 0.8f, 0.1f}, {1, 1, 0}};
  for (float T : {0.0f, 1.0f, 0.6f})
    for (const Filt& f : filts) {
      const int32_t k = std::min<int32_t>(f.k, (int32_t)vocab);
      expect_ok(oracle_spec_accept(t.data(), ld, d.data(), ld, B, G, vocab, T, k, f.tp, f.mp, toks.data(), ua.data(),
                                   ur.data(), ub.data(), lm.data(), tm.data(), la.data(), ta.data(), smin.data(),
                                   am.data(), dm.data(), fm.data(), threads),
                "spec_accept");
      expect_ok(oracle_spec_match(t.data(), ld, d.data(), ld, B, G, vocab, T, k, f.tp, f.mp, toks.data(), um.data(),
                                  ls.data(), tsm.data(), sprod.data(), mm.data(), fm2.data(), threads),
                "spec_match");
    }
}

}  // namespace

int main() {
  int64_t c = 0, tail = 0;
  oracle_chunk_geometry(202048, 1024, &c, &tail);
  if (c != 198 || tail != 320) ++failures;
  for (int threads : {1, 4}) {
    selection(7, 1, 1, threads);
    selection(7, 9, 12, threads);
    selection(14, 1000, 1003, threads);
    selection(7, 20011, 20011, threads);
    speculative(1, 1, 2, threads);
    speculative(5, 3, 7, threads);
    speculative(6, 4, 3000, threads);
  }
  std::printf("oracle driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
