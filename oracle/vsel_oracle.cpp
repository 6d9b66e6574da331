// vsel_oracle.cpp -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, obviously-correct CPU implementation of vocab-row selection,
// used as the parity oracle for the GPU library.  Only the test suite, the
// smoke check and the benchmark's CPU-baseline leg may load it; the product
// path never calls it.  It shares no code, header or constant with the GPU
// library.
//
// Conventions (all functions):
//   * A row is `vocab` valid elements at stride `ld` elements.  dtype 0 is
//     IEEE float32; dtype 1 is bfloat16, widened exactly by placing its 16
//     bits in the top half of a float32.
//   * Comparisons are plain float comparisons, so -0.0 == +0.0 and ties are
//     broken by the lower index.  All arithmetic on values is float64.
//   * A row that holds a NaN or +inf "fails closed": its index output is
//     0xFFFFFFFF, never a token.  -inf is a legal mask value.
//   * Work is split over rows only (std::thread); within a row every loop
//     runs in index order.
//
// Parity pins: every function here is checked in tests/test_oracle_pins.py
// against facts the pages and the mathematics fix (closed forms, library
// routines, brute force on tiny inputs, exact-rational acceptance sums).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t kFailClosed = 0xFFFFFFFFu;
constexpr double kInf = std::numeric_limits<double>::infinity();
constexpr double kNaN = std::numeric_limits<double>::quiet_NaN();

struct Rows {
  const void* base;
  int dtype;
  int64_t ld;
  // Exact element value as float32.
  float at(int64_t r, int64_t i) const {
    if (dtype == 0) {
      float f;
      std::memcpy(&f, static_cast<const char*>(base) + 4 * (r * ld + i), 4);
      return f;
    }
    uint16_t h;
    std::memcpy(&h, static_cast<const char*>(base) + 2 * (r * ld + i), 2);
    uint32_t u = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
};

template <class F>
void for_rows(int64_t n, int nthreads, F fn) {
  if (nthreads <= 0) nthreads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  if (nthreads > n) nthreads = static_cast<int>(std::max<int64_t>(1, n));
  if (nthreads == 1) {
    for (int64_t r = 0; r < n; ++r) fn(r);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < nthreads; ++t)
    pool.emplace_back([&, t] {
      for (int64_t r = t; r < n; r += nthreads) fn(r);
    });
  for (auto& th : pool) th.join();
}

bool is_bad(float x) { return std::isnan(x) || x == std::numeric_limits<float>::infinity(); }

// First-maximum scan: strictly greater, so ties keep the lower index
// ("Chapter 21", section 21.3, and the CPU first-maximum helper with its
// finite-check described in section 21.6).  Returns the index or kFailClosed.
uint32_t argmax_row(const Rows& R, int64_t r, int64_t V, float* best_out) {
  float best = -std::numeric_limits<float>::infinity();
  uint32_t idx = 0;
  bool bad = false;
  for (int64_t i = 0; i < V; ++i) {
    float x = R.at(r, i);
    if (is_bad(x)) bad = true;
    if (x > best) {
      best = x;
      idx = static_cast<uint32_t>(i);
    }
  }
  if (best_out) *best_out = bad ? std::numeric_limits<float>::quiet_NaN() : best;
  if (bad || best == -std::numeric_limits<float>::infinity()) return kFailClosed;
  return idx;
}

bool row_bad(const Rows& R, int64_t r, int64_t V) {
  for (int64_t i = 0; i < V; ++i)
    if (is_bad(R.at(r, i))) return true;
  return false;
}

// log sum_i exp(x_i / T), float64, with M = max_i x_i/T factored out; -inf
// terms contribute nothing.  NaN for a fail-closed row, -inf for an all -inf row.
double lse_row(const Rows& R, int64_t r, int64_t V, double T) {
  if (row_bad(R, r, V)) return kNaN;
  double M = -kInf;
  for (int64_t i = 0; i < V; ++i) M = std::max(M, static_cast<double>(R.at(r, i)) / T);
  if (M == -kInf) return -kInf;
  double s = 0.0;
  for (int64_t i = 0; i < V; ++i) s += std::exp(static_cast<double>(R.at(r, i)) / T - M);
  return M + std::log(s);
}

// A verify row's effective distribution ("speculative-acceptance.md", "The
// rules": top-k / top-p / min-p filtering on the untempered distribution, then
// the final temperature scaling): p(x) = exp(z_x / T - lse) on the kept ids,
// 0 elsewhere.  Filters, in this order, each keeping at least one id:
//   top_k > 0: the top_k largest under (value desc, id asc);
//   top_p < 1: in that order, the shortest prefix whose cumulative untempered
//     probability (softmax of the candidates) reaches top_p;
//   min_p > 0: z >= max z + log(min_p) over the candidates.
// No filter: every id kept, lse the whole row's.  `margin` (may be null) gets
// the smaller of the top-p cut's distance to the nearer cumulative sum and the
// min-p threshold's distance to the nearest candidate value (+inf if none).
struct RowDist {
  std::vector<char> keep;  // empty: every id kept
  double lse = 0.0;
  bool kept(int64_t x) const { return keep.empty() || keep[static_cast<size_t>(x)]; }
};
RowDist row_dist(const Rows& R, int64_t r, int64_t V, double T, int32_t top_k, float top_p, float min_p,
                 double* margin) {
  RowDist d;
  if (margin) *margin = kInf;
  if (top_k <= 0 && top_p >= 1.0f && min_p <= 0.0f) {
    d.lse = lse_row(R, r, V, T);
    return d;
  }
  auto z = [&](uint32_t x) { return static_cast<double>(R.at(r, x)); };
  std::vector<uint32_t> cand(static_cast<size_t>(V));
  std::iota(cand.begin(), cand.end(), 0u);
  if (top_k > 0 || top_p < 1.0f) {
    auto by_value = [&](uint32_t a, uint32_t b) { return z(a) > z(b) || (z(a) == z(b) && a < b); };
    const size_t k = top_k > 0 ? std::min<size_t>(static_cast<size_t>(top_k), cand.size()) : cand.size();
    std::partial_sort(cand.begin(), cand.begin() + k, cand.end(), by_value);
    cand.resize(k);
  }
  double zmax = -kInf;
  for (uint32_t x : cand) zmax = std::max(zmax, z(x));
  if (top_p < 1.0f) {
    double Z = 0.0;
    for (uint32_t x : cand) Z += std::exp(z(x) - zmax);
    double cum = 0.0;
    for (size_t j = 0; j < cand.size(); ++j) {
      const double prev = cum;
      cum += std::exp(z(cand[j]) - zmax) / Z;
      if (cum >= static_cast<double>(top_p)) {
        if (margin) *margin = std::min(*margin, std::min(cum - top_p, j > 0 ? top_p - prev : kInf));
        cand.resize(j + 1);
        break;
      }
    }
  }
  if (min_p > 0.0f) {
    const double thr = zmax + std::log(static_cast<double>(min_p));
    std::vector<uint32_t> kept;
    for (uint32_t x : cand) {
      if (z(x) >= thr) kept.push_back(x);
      if (margin) *margin = std::min(*margin, std::fabs(z(x) - thr));
    }
    cand.swap(kept);
  }
  d.keep.assign(static_cast<size_t>(V), 0);
  double M = -kInf;
  for (uint32_t x : cand) {
    d.keep[x] = 1;
    M = std::max(M, z(x) / T);
  }
  double s = 0.0;
  for (uint32_t x : cand) s += std::exp(z(x) / T - M);
  d.lse = M + std::log(s);
  return d;
}

// The effective distributions of one sequence: target rows zrow0 .. +G (the
// last is the bonus row) and draft rows drow0 .. +G-1, all under the same
// sampler settings.  Returns the smallest filter margin.
double seq_dists(const Rows& Zr, int64_t zrow0, const Rows& Dr, int64_t drow0, int64_t G, int64_t V, double T,
                 int32_t top_k, float top_p, float min_p, std::vector<RowDist>& dp, std::vector<RowDist>& dq) {
  dp.resize(static_cast<size_t>(G + 1));
  dq.resize(static_cast<size_t>(G));
  double fm = kInf, m;
  for (int64_t i = 0; i <= G; ++i) {
    dp[i] = row_dist(Zr, zrow0 + i, V, T, top_k, top_p, min_p, &m);
    fm = std::min(fm, m);
  }
  for (int64_t i = 0; i < G; ++i) {
    dq[i] = row_dist(Dr, drow0 + i, V, T, top_k, top_p, min_p, &m);
    fm = std::min(fm, m);
  }
  return fm;
}

// The k first elements of the row under the total order
//   a before b  <=>  x_a > x_b, or x_a == x_b and a < b.
std::vector<uint32_t> topk_row(const Rows& R, int64_t r, int64_t V, int64_t k) {
  std::vector<uint32_t> order(static_cast<size_t>(V));
  std::iota(order.begin(), order.end(), 0u);
  std::partial_sort(order.begin(), order.begin() + k, order.end(), [&](uint32_t a, uint32_t b) {
    float xa = R.at(r, a), xb = R.at(r, b);
    if (xa > xb) return true;
    if (xa < xb) return false;
    return a < b;
  });
  order.resize(static_cast<size_t>(k));
  return order;
}

// Inverse-CDF draw over non-negative weights w (in the given order): the
// first j with u*W < w_0 + ... + w_j, W = sum of all weights (sequential
// float64 sums).  If none (rounding), the last j with w_j > 0.  `margin` is
// the distance of u*W to the nearer boundary of the chosen interval, over W.
size_t draw(const std::vector<double>& w, double u, double* margin) {
  double W = 0.0;
  for (double x : w) W += x;
  double target = u * W;
  double c = 0.0;
  for (size_t j = 0; j < w.size(); ++j) {
    double prev = c;
    c += w[j];
    if (target < c) {
      if (margin) *margin = std::min(target - prev, c - target) / W;
      return j;
    }
  }
  if (margin) *margin = 0.0;
  for (size_t j = w.size(); j-- > 0;)
    if (w[j] > 0.0) return j;
  return 0;
}

}  // namespace

extern "C" {

// Chunk geometry of a chunked reduction: ceil(n / chunk) chunks, the last
// holding n - (count-1)*chunk elements ("Chapter 21", Figure 21.1).
void oracle_chunk_geometry(int64_t n, int64_t chunk, int64_t* count, int64_t* tail) {
  *count = (n + chunk - 1) / chunk;
  *tail = n - (*count - 1) * chunk;
}

// c1: per-row first-maximum argmax.  out_val (optional) gets the maximum
// value (NaN for a fail-closed row).
int oracle_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                  uint32_t* out_idx, float* out_val, int nthreads) {
  if (!logits || !out_idx || rows < 0 || vocab < 1 || ld < vocab || (dtype != 0 && dtype != 1)) return 1;
  Rows R{logits, dtype, ld};
  for_rows(rows, nthreads, [&](int64_t r) {
    float best;
    out_idx[r] = argmax_row(R, r, vocab, &best);
    if (out_val) out_val[r] = best;
  });
  return 0;
}

// Greedy serving variant ("Chapter 21", section 21.4): the first-maximum
// argmax with the request's excluded ids (its end-of-generation set) taken
// as -inf inside the reduction only -- the row itself is not modified.  A
// NaN or +inf anywhere in the row, excluded or not, fails it closed.  Ids at
// or past vocab exclude nothing.  out_status: 0 ok, 1 nonfinite, 2 no
// element above -inf; out_idx is 0xFFFFFFFF whenever the status is not 0.
int oracle_argmax_excluding(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                            const uint32_t* excluded, int64_t n_excluded, uint32_t* out_idx,
                            uint32_t* out_status, int nthreads) {
  if (!logits || !out_idx || !out_status || rows < 0 || vocab < 1 || ld < vocab || n_excluded < 0 ||
      (n_excluded > 0 && !excluded) || (dtype != 0 && dtype != 1))
    return 1;
  std::vector<char> is_excluded(static_cast<size_t>(vocab), 0);
  for (int64_t j = 0; j < n_excluded; ++j)
    if (excluded[j] < static_cast<uint64_t>(vocab)) is_excluded[excluded[j]] = 1;
  Rows R{logits, dtype, ld};
  const float neg_inf = -std::numeric_limits<float>::infinity();
  for_rows(rows, nthreads, [&](int64_t r) {
    float best = neg_inf;
    uint32_t idx = 0;
    bool bad = false;
    for (int64_t i = 0; i < vocab; ++i) {
      const float x = R.at(r, i);
      if (is_bad(x)) bad = true;
      const float v = is_excluded[i] ? neg_inf : x;
      if (v > best) {
        best = v;
        idx = static_cast<uint32_t>(i);
      }
    }
    const uint32_t status = bad ? 1u : (best == neg_inf ? 2u : 0u);
    out_status[r] = status;
    out_idx[r] = status ? kFailClosed : idx;
  });
  return 0;
}

// c3: per-row log-sum-exp at temperature T > 0, float64.
int oracle_lse(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
               double temperature, double* out_lse, int nthreads) {
  if (!logits || !out_lse || rows < 0 || vocab < 1 || ld < vocab || !(temperature > 0.0)) return 1;
  Rows R{logits, dtype, ld};
  for_rows(rows, nthreads, [&](int64_t r) { out_lse[r] = lse_row(R, r, vocab, temperature); });
  return 0;
}

// c2: exact top-k (value, id) pairs per row in (value desc, id asc) order,
// with the row's argmax and log-sum-exp at T = 1 (both optional).  A
// fail-closed row gets ids[0] = 0xFFFFFFFF (its other entries are filled
// with 0xFFFFFFFF / NaN).  Values are the row's own elements, widened exactly.
int oracle_topk(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k,
                float* out_vals, uint32_t* out_ids, uint32_t* out_argmax, double* out_lse,
                int nthreads) {
  if (!logits || !out_vals || !out_ids || rows < 0 || vocab < 1 || ld < vocab || k < 1 || k > vocab)
    return 1;
  Rows R{logits, dtype, ld};
  for_rows(rows, nthreads, [&](int64_t r) {
    if (out_argmax) out_argmax[r] = argmax_row(R, r, vocab, nullptr);
    if (out_lse) out_lse[r] = lse_row(R, r, vocab, 1.0);
    if (row_bad(R, r, vocab)) {
      for (int32_t j = 0; j < k; ++j) {
        out_ids[r * k + j] = kFailClosed;
        out_vals[r * k + j] = std::numeric_limits<float>::quiet_NaN();
      }
      return;
    }
    std::vector<uint32_t> ids = topk_row(R, r, vocab, k);
    for (int32_t j = 0; j < k; ++j) {
      out_ids[r * k + j] = ids[j];
      out_vals[r * k + j] = R.at(r, ids[j]);
    }
  });
  return 0;
}

// c4: temperature sampling with top-k then top-p, one caller uniform per row.
//   1. T == 0 or top_k == 1: the argmax token, logp = 0, nothing drawn.
//   2. candidates c_0..c_{k-1}: top-k of the raw logits (k = min(top_k, V));
//      top_k == 0 means the whole row in id order and then requires top_p == 1.
//   3. untempered p0_j = exp(z_j - z_0) / sum_i exp(z_i - z_0) over candidates.
//   4. top-p: keep the first n >= 1 candidates, n the smallest with
//      p0_0 + ... + p0_{n-1} >= top_p (n = k when top_p >= 1).
//   5. temperature last: w_j = exp((z_j - z_0) / T) over the kept set.
//   6. inverse-CDF draw with u in candidate order; logp = log(w_j / sum w).
// Filters act on the untempered distribution and the temperature is applied
// last ("speculative-acceptance.md", "The rules", definition of p).
// margins (optional, 2 per row): [0] the draw margin over the total weight,
// [1] the distance of top_p to the nearer cumulative sum at the top-p cut.
int oracle_sample(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                  float temperature, int32_t top_k, float top_p, const float* u,
                  uint32_t* out_token, double* out_logp, double* margins, int nthreads) {
  if (!logits || !u || !out_token || rows < 0 || vocab < 1 || ld < vocab) return 1;
  if (!(temperature >= 0.0f) || top_k < 0 || !(top_p > 0.0f && top_p <= 1.0f)) return 1;
  if (top_k == 0 && top_p < 1.0f) return 1;
  Rows R{logits, dtype, ld};
  const double T = temperature, P = top_p;
  for_rows(rows, nthreads, [&](int64_t r) {
    double m_draw = kInf, m_topp = kInf;
    auto finish = [&](uint32_t tok, double logp) {
      out_token[r] = tok;
      if (out_logp) out_logp[r] = logp;
      if (margins) {
        margins[2 * r] = m_draw;
        margins[2 * r + 1] = m_topp;
      }
    };
    uint32_t am = argmax_row(R, r, vocab, nullptr);
    if (am == kFailClosed) return finish(kFailClosed, kNaN);
    if (temperature == 0.0f || top_k == 1) return finish(am, 0.0);
    std::vector<uint32_t> cand;
    if (top_k == 0) {
      cand.resize(static_cast<size_t>(vocab));
      std::iota(cand.begin(), cand.end(), 0u);
    } else {
      cand = topk_row(R, r, vocab, std::min<int64_t>(top_k, vocab));
    }
    const size_t k = cand.size();
    const double z0 = R.at(r, am);  // the row maximum (the first candidate when sorted)
    size_t n = k;
    if (P < 1.0) {
      std::vector<double> e(k);
      double Z0 = 0.0;
      for (size_t j = 0; j < k; ++j) Z0 += (e[j] = std::exp(static_cast<double>(R.at(r, cand[j])) - z0));
      double cum = 0.0, prev = 0.0;
      n = 0;
      for (size_t j = 0; j < k; ++j) {
        prev = cum;
        cum += e[j] / Z0;
        if (cum >= P) {
          n = j + 1;
          m_topp = std::min(cum - P, j > 0 ? P - prev : kInf);
          break;
        }
      }
      if (n == 0) n = k;
    }
    std::vector<double> w(n);
    for (size_t j = 0; j < n; ++j) w[j] = std::exp((static_cast<double>(R.at(r, cand[j])) - z0) / T);
    size_t j = draw(w, static_cast<double>(u[r]), &m_draw);
    double S = 0.0;
    for (double x : w) S += x;
    finish(cand[j], (static_cast<double>(R.at(r, cand[j])) - z0) / T - std::log(S));
  });
  return 0;
}

// f3: the ordered sampler chain ("Chapter 21", section 21.7: in source order
// top_n_sigma masking against the maximum, top_k truncation, typical_p, then
// the top_p nucleus cutoff, each over the full candidate list; min_p among the
// filters on the untempered distribution, and the temperature last:
// "speculative-acceptance.md", "The rules").  Candidates start as the whole
// row in id order; every filter keeps at least one.
//   1. top_n_sigma > 0: keep z >= z_max - n * sigma, sigma the population
//      standard deviation of the row's values above -inf (order unchanged);
//   2. top_k > 0: the top_k largest (value desc, id asc), in that order;
//   3. typical_p < 1: p = softmax of the candidates (untempered), H = -sum p
//      log p; reorder by |-log p - H| ascending (ties keep the current order),
//      keep the shortest prefix with sum p >= typical_p;
//   4. top_p < 1: reorder by (value desc, id asc), keep the shortest prefix
//      with sum p >= top_p, p the softmax of the current candidates;
//   5. min_p > 0: keep p >= min_p * max p over the candidates, i.e.
//      z >= z_max + log(min_p) (order unchanged);
//   6. w = exp((z - z_max) / T) over the kept candidates, the inverse-CDF draw
//      with u in their current order, logp = log(w_j / sum w).
// T == 0 or top_k == 1: the argmax, logp 0 (nothing drawn).
// margins (6 per row, +inf when not applicable): the draw margin over W; the
// distance of typical_p / top_p to the nearer cumulative sum at its cut; the
// distance of the top-n-sigma and min-p thresholds to the nearest candidate
// value (logit units); the smallest gap between the typicality scores of the
// typical cut's element, or of the element drawn in typical order, and its
// neighbours in that order, relative to the larger score or to 1 when both
// are below 1 (elements of equal value excluded).
int oracle_sample_chain(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                        float temperature, float top_n_sigma, int32_t top_k, float typical_p, float top_p,
                        float min_p, const float* u, uint32_t* out_token, double* out_logp, double* margins,
                        int nthreads) {
  if (!logits || !u || !out_token || rows < 0 || vocab < 1 || ld < vocab) return 1;
  if (!(temperature >= 0.0f) || top_k < 0 || !(top_p > 0.0f && top_p <= 1.0f) ||
      !(typical_p > 0.0f && typical_p <= 1.0f) || !(min_p >= 0.0f && min_p <= 1.0f) || !(top_n_sigma >= 0.0f))
    return 1;
  Rows R{logits, dtype, ld};
  const double T = temperature;
  for_rows(rows, nthreads, [&](int64_t r) {
    double mg[6] = {kInf, kInf, kInf, kInf, kInf, kInf};
    auto finish = [&](uint32_t tok, double logp) {
      out_token[r] = tok;
      if (out_logp) out_logp[r] = logp;
      if (margins)
        for (int q = 0; q < 6; ++q) margins[6 * r + q] = mg[q];
    };
    const uint32_t am = argmax_row(R, r, vocab, nullptr);
    if (am == kFailClosed) return finish(kFailClosed, kNaN);
    if (temperature == 0.0f || top_k == 1) return finish(am, 0.0);
    auto z = [&](uint32_t x) { return static_cast<double>(R.at(r, x)); };
    const double zmax = z(am);
    std::vector<uint32_t> cand(static_cast<size_t>(vocab));
    std::iota(cand.begin(), cand.end(), 0u);
    // 1. top-n-sigma
    if (top_n_sigma > 0.0f) {
      double n = 0.0, mean = 0.0;
      for (uint32_t x : cand)
        if (z(x) > -kInf) {
          n += 1.0;
          mean += z(x);
        }
      mean /= n;
      double var = 0.0;
      for (uint32_t x : cand)
        if (z(x) > -kInf) var += (z(x) - mean) * (z(x) - mean);
      const double thr = zmax - static_cast<double>(top_n_sigma) * std::sqrt(var / n);
      std::vector<uint32_t> kept;
      for (uint32_t x : cand) {
        if (z(x) >= thr) kept.push_back(x);
        mg[3] = std::min(mg[3], std::fabs(z(x) - thr));
      }
      cand.swap(kept);
    }
    auto by_value = [&](uint32_t a, uint32_t b) { return z(a) > z(b) || (z(a) == z(b) && a < b); };
    // 2. top-k
    if (top_k > 0) {
      const size_t k = std::min<size_t>(static_cast<size_t>(top_k), cand.size());
      std::partial_sort(cand.begin(), cand.begin() + k, cand.end(), by_value);
      cand.resize(k);
    }
    // untempered softmax of the current candidates (relative to zmax: cancels)
    auto probs = [&](std::vector<double>& p) {
      p.resize(cand.size());
      double Z = 0.0;
      for (size_t j = 0; j < cand.size(); ++j) Z += (p[j] = std::exp(z(cand[j]) - zmax));
      for (double& v : p) v /= Z;
    };
    // shortest prefix of the current order with cumulative p >= P (at least 1)
    auto cut = [&](const std::vector<double>& p, double P, double* margin) {
      double cum = 0.0;
      for (size_t j = 0; j < p.size(); ++j) {
        const double prev = cum;
        cum += p[j];
        if (cum >= P) {
          *margin = std::min(cum - P, j > 0 ? P - prev : kInf);
          cand.resize(j + 1);
          return;
        }
      }
    };
    // 3. typical-p
    // tscore: each candidate's typicality score, kept for the near-tie margin
    std::vector<double> tscore;
    // score gap of two ids, relative to the larger score or to one logit unit
    // when both are smaller (+inf for equal values, which tie exactly)
    auto tgap = [&](uint32_t a, uint32_t b) {
      if (z(a) == z(b)) return kInf;
      const double sa = tscore[a], sb = tscore[b];
      return std::fabs(sa - sb) / std::max(std::max(sa, sb), 1.0);
    };
    if (typical_p < 1.0f) {
      std::vector<double> p;
      probs(p);
      double H = 0.0;
      for (double v : p)
        if (v > 0.0) H -= v * std::log(v);
      std::vector<size_t> idx(cand.size());
      std::iota(idx.begin(), idx.end(), size_t(0));
      auto score = [&](size_t j) { return p[j] > 0.0 ? std::fabs(-std::log(p[j]) - H) : kInf; };
      std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return score(a) < score(b); });
      std::vector<uint32_t> c2(cand.size());
      std::vector<double> p2(cand.size());
      tscore.assign(static_cast<size_t>(vocab), kInf);
      for (size_t j = 0; j < idx.size(); ++j) {
        c2[j] = cand[idx[j]];
        p2[j] = p[idx[j]];
        tscore[c2[j]] = score(idx[j]);
      }
      cand.swap(c2);
      const std::vector<uint32_t> full = cand;
      cut(p2, typical_p, &mg[1]);
      // near-ties of the typical order beside the cut (an order taken in
      // float32 scores may swap them)
      const size_t jc = cand.size() - 1;
      if (jc + 1 < full.size()) mg[5] = std::min(mg[5], tgap(full[jc], full[jc + 1]));
      if (jc > 0) mg[5] = std::min(mg[5], tgap(full[jc], full[jc - 1]));
    }
    // 4. top-p
    if (top_p < 1.0f) {
      std::sort(cand.begin(), cand.end(), by_value);
      std::vector<double> p;
      probs(p);
      cut(p, top_p, &mg[2]);
    }
    // 5. min-p
    if (min_p > 0.0f) {
      double cmax = -kInf;
      for (uint32_t x : cand) cmax = std::max(cmax, z(x));
      const double thr = cmax + std::log(static_cast<double>(min_p));
      std::vector<uint32_t> kept;
      for (uint32_t x : cand) {
        if (z(x) >= thr) kept.push_back(x);
        mg[4] = std::min(mg[4], std::fabs(z(x) - thr));
      }
      cand.swap(kept);
    }
    // 6. temperature, then the draw in the current order
    std::vector<double> w(cand.size());
    for (size_t j = 0; j < cand.size(); ++j) w[j] = std::exp((z(cand[j]) - zmax) / T);
    const size_t j = draw(w, static_cast<double>(u[r]), &mg[0]);
    if (typical_p < 1.0f && top_p >= 1.0f) {  // the draw ran in typical order: near-ties beside it
      if (j + 1 < cand.size()) mg[5] = std::min(mg[5], tgap(cand[j], cand[j + 1]));
      if (j > 0) mg[5] = std::min(mg[5], tgap(cand[j], cand[j - 1]));
    }
    double S = 0.0;
    for (double v : w) S += v;
    finish(cand[j], (z(cand[j]) - zmax) / T - std::log(S));
  });
  return 0;
}

// c5: speculative acceptance for `batch` sequences of `gamma` drafted tokens.
// target: batch*(gamma+1) rows (row b*(gamma+1)+i is verify position i of
// sequence b; the last one is the bonus row); draft: batch*gamma rows.
//   p_i = softmax(Z_i / T), q_i = softmax(D_i / T), float64 via log-sum-exp;
//   with filters (top_k, top_p, min_p: row_dist) both are the filtered,
//   renormalised distributions, the same sampler settings on target and draft.
//   Modified rejection sampling ("speculative-acceptance.md", "Modified
//   rejection sampling"; the exact CPU acceptance of "Chapter 21", section
//   21.9): accept t_i iff u_acc * q_i(t_i) <= p_i(t_i) (q = 0 accepts); at the
//   first rejection L draw once from normalize(max(p_L - q_L, 0)) with u_res
//   (from p_L when that residual sums to <= 0); if all gamma are accepted draw
//   the bonus token from p_gamma with u_bon.  Draws run in id order.
//   Argmax-against-argmax: accept iff t_i == argmax(Z_i); emit that argmax at
//   the first mismatch (or argmax(Z_gamma) when all match).
//   summin[b*gamma+i] = sum_x min(p_i(x), q_i(x)) for every position.
//   T == 0 is greedy: both rules are argmax-against-argmax and summin is 1
//   where the two argmaxes agree, else 0.
// Outputs: len = accepted drafts L (0..gamma) or -1 for a fail-closed
// sequence (any nonfinite row used by it, or a drafted id >= vocab);
// tokens[b*(gamma+1) + 0..L] emitted, the rest 0xFFFFFFFF.
// Margins (optional): acc_margin[b*gamma+i] = |u_acc*q_i(t_i) - p_i(t_i)| for
// tested positions (+inf elsewhere); draw_margin[b] as in draw();
// filter_margin[b] the smallest row_dist margin over the sequence's rows.
int oracle_spec_accept(const float* target, int64_t ld_t, const float* draft, int64_t ld_d,
                       int64_t batch, int32_t gamma, int64_t vocab, float temperature, int32_t top_k,
                       float top_p, float min_p, const uint32_t* draft_tokens, const float* u_acc,
                       const float* u_res, const float* u_bon, int32_t* len_mrs, uint32_t* tok_mrs,
                       int32_t* len_aa, uint32_t* tok_aa, double* summin, double* acc_margin,
                       double* draw_margin, double* filter_margin, int nthreads) {
  if (!target || !draft || !draft_tokens || !u_acc || !u_res || !u_bon || !len_mrs || !tok_mrs) return 1;
  if (batch < 0 || gamma < 1 || vocab < 1 || ld_t < vocab || ld_d < vocab || !(temperature >= 0.0f)) return 1;
  if (top_k < 0 || !(top_p > 0.0f && top_p <= 1.0f) || !(min_p >= 0.0f && min_p <= 1.0f)) return 1;
  Rows Zr{target, 0, ld_t}, Dr{draft, 0, ld_d};
  const int64_t G = gamma, V = vocab;
  const double T = temperature;
  for_rows(batch, nthreads, [&](int64_t b) {
    const int64_t zrow0 = b * (G + 1), drow0 = b * G;
    uint32_t* tm = tok_mrs + b * (G + 1);
    uint32_t* ta = tok_aa ? tok_aa + b * (G + 1) : nullptr;
    for (int64_t i = 0; i <= G; ++i) {
      tm[i] = kFailClosed;
      if (ta) ta[i] = kFailClosed;
    }
    for (int64_t i = 0; i < G; ++i) {
      if (acc_margin) acc_margin[b * G + i] = kInf;
      if (summin) summin[b * G + i] = kNaN;
    }
    if (draw_margin) draw_margin[b] = kInf;
    if (filter_margin) filter_margin[b] = kInf;
    auto fail = [&] {
      len_mrs[b] = -1;
      if (len_aa) len_aa[b] = -1;
    };
    // Fail closed on any nonfinite (or all -inf) row and on out-of-range drafts.
    std::vector<uint32_t> amz(G + 1), amd(G);
    for (int64_t i = 0; i <= G; ++i)
      if ((amz[i] = argmax_row(Zr, zrow0 + i, V, nullptr)) == kFailClosed) return fail();
    for (int64_t i = 0; i < G; ++i)
      if ((amd[i] = argmax_row(Dr, drow0 + i, V, nullptr)) == kFailClosed) return fail();
    for (int64_t i = 0; i < G; ++i)
      if (draft_tokens[b * G + i] >= V) return fail();

    // Argmax-against-argmax.
    int64_t Laa = G;
    for (int64_t i = 0; i < G; ++i)
      if (draft_tokens[b * G + i] != amz[i]) {
        Laa = i;
        break;
      }
    if (len_aa) len_aa[b] = static_cast<int32_t>(Laa);
    if (ta) {
      for (int64_t i = 0; i < Laa; ++i) ta[i] = draft_tokens[b * G + i];
      ta[Laa] = amz[Laa];
    }

    if (temperature == 0.0f) {
      len_mrs[b] = static_cast<int32_t>(Laa);
      for (int64_t i = 0; i < Laa; ++i) tm[i] = draft_tokens[b * G + i];
      tm[Laa] = amz[Laa];
      if (summin)
        for (int64_t i = 0; i < G; ++i) summin[b * G + i] = (amz[i] == amd[i]) ? 1.0 : 0.0;
      return;
    }

    std::vector<RowDist> dp, dq;
    const double fm = seq_dists(Zr, zrow0, Dr, drow0, G, V, T, top_k, top_p, min_p, dp, dq);
    if (filter_margin) filter_margin[b] = fm;
    auto p_of = [&](int64_t i, int64_t x) {
      return dp[i].kept(x) ? std::exp(static_cast<double>(Zr.at(zrow0 + i, x)) / T - dp[i].lse) : 0.0;
    };
    auto q_of = [&](int64_t i, int64_t x) {
      return dq[i].kept(x) ? std::exp(static_cast<double>(Dr.at(drow0 + i, x)) / T - dq[i].lse) : 0.0;
    };

    if (summin)
      for (int64_t i = 0; i < G; ++i) {
        double s = 0.0;
        for (int64_t x = 0; x < V; ++x) s += std::min(p_of(i, x), q_of(i, x));
        summin[b * G + i] = s;
      }

    int64_t L = G;
    for (int64_t i = 0; i < G; ++i) {
      const uint32_t t = draft_tokens[b * G + i];
      const double pt = p_of(i, t), qt = q_of(i, t);
      const double lhs = static_cast<double>(u_acc[b * G + i]) * qt;
      if (acc_margin) acc_margin[b * G + i] = std::fabs(lhs - pt);
      if (!(lhs <= pt)) {
        L = i;
        break;
      }
    }
    std::vector<double> w(static_cast<size_t>(V));
    double u;
    if (L < G) {
      double W = 0.0;
      for (int64_t x = 0; x < V; ++x) W += (w[x] = std::max(p_of(L, x) - q_of(L, x), 0.0));
      if (W <= 0.0)
        for (int64_t x = 0; x < V; ++x) w[x] = p_of(L, x);
      u = u_res[b * G + L];
    } else {
      for (int64_t x = 0; x < V; ++x) w[x] = p_of(G, x);
      u = u_bon[b];
    }
    double m;
    size_t x = draw(w, u, &m);
    if (draw_margin) draw_margin[b] = m;
    len_mrs[b] = static_cast<int32_t>(L);
    for (int64_t i = 0; i < L; ++i) tm[i] = draft_tokens[b * G + i];
    tm[L] = static_cast<uint32_t>(x);
  });
  return 0;
}

// f1: sampler-match ("speculative-acceptance.md", "The rules": the default
// rule at T > 0).  At each verify position i = 0, 1, ... a fresh draw x_i
// from p_i (id order, as draw()) with u_match[b*(gamma+1) + i]; the drafted
// t_i is accepted iff x_i == t_i, and the chain ends at the first mismatch L
// (or at gamma, where x_gamma is drawn from the bonus row p_gamma), emitting
// t_0 .. t_{L-1}, x_L: the draw is emitted on both branches, so every
// emitted token is a draw from the target.
//   sumprod[b*gamma+i] = sum_x p_i(x) q_i(x) for every position: the rule's
//   acceptance probability for a proposal drawn from q ("The acceptance
//   ceiling", the sampler-match row), the diagnostic beside sum min(p, q).
//   T == 0 is greedy: the sampler is argmax, so the rule is
//   argmax-against-argmax, and sumprod is 1 where the two argmaxes agree.
// p and q filtered as in oracle_spec_accept.  Outputs as oracle_spec_accept
// (len -1 and sentinel tokens for a fail-closed sequence).
// match_margin[b*(gamma+1)+i]: the draw margin at every position the chain
// tested (+inf elsewhere); filter_margin as in oracle_spec_accept.
int oracle_spec_match(const float* target, int64_t ld_t, const float* draft, int64_t ld_d, int64_t batch,
                      int32_t gamma, int64_t vocab, float temperature, int32_t top_k, float top_p, float min_p,
                      const uint32_t* draft_tokens, const float* u_match, int32_t* len_sm, uint32_t* tok_sm,
                      double* sumprod, double* match_margin, double* filter_margin, int nthreads) {
  if (!target || !draft || !draft_tokens || !u_match || !len_sm || !tok_sm) return 1;
  if (batch < 0 || gamma < 1 || vocab < 1 || ld_t < vocab || ld_d < vocab || !(temperature >= 0.0f)) return 1;
  if (top_k < 0 || !(top_p > 0.0f && top_p <= 1.0f) || !(min_p >= 0.0f && min_p <= 1.0f)) return 1;
  Rows Zr{target, 0, ld_t}, Dr{draft, 0, ld_d};
  const int64_t G = gamma, V = vocab;
  const double T = temperature;
  for_rows(batch, nthreads, [&](int64_t b) {
    const int64_t zrow0 = b * (G + 1), drow0 = b * G;
    uint32_t* tk = tok_sm + b * (G + 1);
    for (int64_t i = 0; i <= G; ++i) {
      tk[i] = kFailClosed;
      if (match_margin) match_margin[b * (G + 1) + i] = kInf;
    }
    for (int64_t i = 0; i < G; ++i)
      if (sumprod) sumprod[b * G + i] = kNaN;
    if (filter_margin) filter_margin[b] = kInf;
    std::vector<uint32_t> amz(G + 1), amd(G);
    for (int64_t i = 0; i <= G; ++i)
      if ((amz[i] = argmax_row(Zr, zrow0 + i, V, nullptr)) == kFailClosed) {
        len_sm[b] = -1;
        return;
      }
    for (int64_t i = 0; i < G; ++i)
      if ((amd[i] = argmax_row(Dr, drow0 + i, V, nullptr)) == kFailClosed || draft_tokens[b * G + i] >= V) {
        len_sm[b] = -1;
        return;
      }
    if (temperature == 0.0f) {  // the sampler is argmax
      int64_t L = G;
      for (int64_t i = 0; i < G; ++i)
        if (draft_tokens[b * G + i] != amz[i]) {
          L = i;
          break;
        }
      len_sm[b] = static_cast<int32_t>(L);
      for (int64_t i = 0; i < L; ++i) tk[i] = draft_tokens[b * G + i];
      tk[L] = amz[L];
      if (sumprod)
        for (int64_t i = 0; i < G; ++i) sumprod[b * G + i] = (amz[i] == amd[i]) ? 1.0 : 0.0;
      return;
    }
    std::vector<RowDist> dp, dq;
    const double fm = seq_dists(Zr, zrow0, Dr, drow0, G, V, T, top_k, top_p, min_p, dp, dq);
    if (filter_margin) filter_margin[b] = fm;
    auto p_of = [&](int64_t i, int64_t x) {
      return dp[i].kept(x) ? std::exp(static_cast<double>(Zr.at(zrow0 + i, x)) / T - dp[i].lse) : 0.0;
    };
    auto q_of = [&](int64_t i, int64_t x) {
      return dq[i].kept(x) ? std::exp(static_cast<double>(Dr.at(drow0 + i, x)) / T - dq[i].lse) : 0.0;
    };
    if (sumprod)
      for (int64_t i = 0; i < G; ++i) {
        double s = 0.0;
        for (int64_t x = 0; x < V; ++x) s += p_of(i, x) * q_of(i, x);
        sumprod[b * G + i] = s;
      }
    std::vector<double> w(static_cast<size_t>(V));
    for (int64_t i = 0; i <= G; ++i) {
      for (int64_t x = 0; x < V; ++x) w[x] = p_of(i, x);
      double m;
      const uint32_t x = static_cast<uint32_t>(draw(w, u_match[b * (G + 1) + i], &m));
      if (match_margin) match_margin[b * (G + 1) + i] = m;
      tk[i] = x;
      if (i == G || x != draft_tokens[b * G + i]) {
        len_sm[b] = static_cast<int32_t>(i);
        return;
      }
    }
  });
  return 0;
}

}  // extern "C"
