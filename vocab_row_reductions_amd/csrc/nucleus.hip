// nucleus.hip -- the sampler chain over whole rows with a top-p cut
// ("Chapter 21", section 21.7: top_n_sigma, then the top_p nucleus over the
// candidate list; min_p among the untempered filters and the temperature last,
// "speculative-acceptance.md", "The rules"), for top_k = 0: the candidates are
// the whole row, ordered by (value desc, id asc).
//
// Both decisions of a row are weighted selections in that order:
//   1. the nucleus cut: the first candidate at which the cumulative untempered
//      mass exp(z - max) reaches top_p times the candidates' total;
//   2. the draw: among the kept candidates (the nucleus, narrowed by min_p),
//      the first at which the cumulative tempered mass exp((z - max) / T)
//      passes u times the kept total.
// The row is never sorted.  A guide histogram of the masses (summed in
// float64 in the order the LDS atomics land; 4,096 bins of equal steps of
// (max - z) / T over [0, span), span the crossing bound below, deeper
// candidates sharing the last bin; the parallel passes add the exact weights,
// the one-workgroup refinement float32 exponentials) places a window of
// candidates around the crossing, wider than the guide's error.
// An exact pass then sums the float64 masses above the window and the totals
// in a fixed order and gathers the window's candidates; they are sorted in LDS
// and walked in order.
//
// Four launches, the first three over (row, segment) workgroups, the last
// workgroup of a row finishing it:
//   nuc_hist:    guide histogram of the untempered masses and their exact
//                total, and every segment's candidates short of the last bin
//                gathered into a list of the (row, segment); the last
//                workgroup places the cut window (from the top of the row when
//                everything above the crossing fits LDS) and marks the row
//                "listed" when every list is whole and the window stays short
//                of the last bin.  The later passes of a listed row visit its
//                lists instead of the row.
//   nuc_collect: the exact mass above the window and the window's candidates,
//                and the guide histogram and exact mass of the tempered
//                weights above it; the last workgroup cuts, applies min_p,
//                totals the kept mass and draws when the draw falls in the
//                window, else places the draw window.
//   nuc_draw:    for the remaining rows, the same over the draw window.
//   nuc_alone:   one workgroup per row, for a window with more candidates than
//                LDS holds: it narrows the window by guide passes over equal
//                steps of the composite key (value, then id); these also
//                separate tied values.
// A window of at most 64 candidates is sorted and walked by one wave in its
// lanes, one of at most 256 by ranks, one per thread.
//
// Typical-p over whole rows (further down) uses the same guide / window /
// fallback scheme for each of its selections, in the typical order or in
// value order, with a per-row job record carrying one selection to the next.
#include "device.hpp"
#include "internal.hpp"

namespace vsel {

// Row `row` of the launch's rows: rows past rows1 belong to the second batch.
template <typename DT>
__device__ __forceinline__ const DT* nuc_row(const NucArgs& a, int64_t row) {
  if (a.x2 != nullptr && row >= a.rows1) return reinterpret_cast<const DT*>(a.x2) + (row - a.rows1) * a.ld2;
  return reinterpret_cast<const DT*>(a.x) + row * a.ld;
}

constexpr int kNB = kNucBins;          // guide bins of the parallel passes
constexpr int kFbNB = 2048;            // guide bins of the one-workgroup refinement
constexpr double kSpan = 40.0;         // (max - z) / T in [0, 40) in equal steps; lower values share the last bin
constexpr uint32_t kCapW = kNucCap;    // window candidates sorted in LDS
constexpr double kGuard = 1e-5;        // window half-width around a target, relative to the total mass
constexpr int kMaxLevels = 12;         // key passes (each narrows the key range by at least 2^11 / 3)
constexpr uint32_t kRun = kCapW / NT;  // sorted window candidates walked per thread
constexpr int kNG = 4;                 // 16-byte groups per lane per tile

// Typicality keys: the float64 distance |z - c| to the typical centre with its
// mantissa cut to 30 bits, as 38 bits (an 8-bit exponent for distances in
// [2^-125, 2^130); smaller ones count as 0, larger ones do not occur), above
// the complemented id in 26 bits (whole-row calls have vocab <= 2^26).  The
// cut is monotone, so the key order is the float64 order of the distances
// except where two differ by less than 2^-30 relative; those tie and fall to
// the lower id.
constexpr int kTypIdBits = 26;
constexpr uint64_t kTypIdMask = (1ull << kTypIdBits) - 1;
constexpr uint64_t kTypScoreMask = (1ull << 38) - 1;
// The cut distance: the float64 d >= 0 with its low 22 mantissa bits cleared
// (0 below 2^-125), monotone in d.
__device__ __forceinline__ double typ_cut(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d) & ~((1ull << 22) - 1);
  return b < ((uint64_t)(1023 - 125) << 52) ? 0.0 : __longlong_as_double((long long)b);
}
// Its 38-bit score: the exponent, biased by 126, above the 30 mantissa bits
// kept (0 for 0).
__device__ __forceinline__ uint64_t typ_score(double dc) {
  const uint64_t b = (uint64_t)__double_as_longlong(dc);
  return b == 0ull ? 0ull : (b >> 22) - ((uint64_t)(1023 - 126) << 30);
}
// The token id a selection key holds.
__device__ __forceinline__ uint32_t key_id(int order, uint64_t key) {
  return order == 0 ? ~(uint32_t)key : (uint32_t)(~key & kTypIdMask);
}

// The candidates of one selection, their order and their weights.
//   order 0: (value desc, id asc), key comp_key;
//   order 1: typicality, (|z - c| asc, id asc), key score_key: the cut
//     float64 distance to the typical centre c above the complemented id.
//   A typical set (kT != 0) keeps the elements whose score key is >= kT.
struct NucSet {
  double m;           // the row maximum
  double thr;         // candidates have z >= thr (and z > -inf)
  uint64_t kfloor;    // ... and order key >= kfloor
  double T;           // weight exp((z - m) / T)
  const double* e2;   // the exp table
  int order;          // 0 value, 1 typicality
  double c;           // typical centre (order 1, typical sets)
  double span;        // first-level bins are equal steps of the bin coordinate over [0, span)
  uint64_t kT;        // typical set: score key >= kT (0: none)
  __device__ __forceinline__ uint64_t score_key_of(double dc, uint32_t i) const {
    return ((~typ_score(dc) & kTypScoreMask) << kTypIdBits) | (~(uint64_t)i & kTypIdMask);
  }
  __device__ __forceinline__ uint64_t score_key(uint32_t bits, uint32_t i) const {
    return score_key_of(typ_cut(fabs((double)__uint_as_float(bits) - c)), i);
  }
  __device__ __forceinline__ uint64_t key(uint32_t bits, uint32_t i) const {
    return order == 0 ? comp_key(bits, i) : score_key(bits, i);
  }
  __device__ __forceinline__ bool in(float z, uint64_t K) const {
    return z > -__builtin_inff() && (double)z >= thr && K >= kfloor;
  }
  __device__ __forceinline__ bool in(uint32_t bits, uint32_t i, uint64_t K) const {
    return in(__uint_as_float(bits), K) && (kT == 0 || score_key(bits, i) >= kT);
  }
  // (z - m) / T as a product with 1 / T (loop-invariant)
  __device__ __forceinline__ double x(float z) const { return T == 1.0 ? (double)z - m : ((double)z - m) * (1.0 / T); }
  __device__ __forceinline__ double w(float z) const { return exp_le0(x(z), e2); }
  // the weight of an element that passes `ok`, else 0: the exponential is
  // taken either way, so element loops stay free of branches and the
  // exponentials of a tile's elements interleave
  __device__ __forceinline__ double w_if(bool ok, float z) const {
    const double e = w(z);  // (0 for z = -inf)
    return ok ? e : 0.0;
  }
  __device__ __forceinline__ float gw(float z) const {
    return __builtin_amdgcn_exp2f((float)(x(z) * 1.4426950408889634));
  }
  // First-level bins: NB equal steps over [0, span) of (m - z) / T (order 0)
  // or of the cut distance (order 1); the last bin also takes everything
  // deeper.  bin_of takes the coordinate already scaled by NB / span (order
  // 0: z - m times the loop-invariant vscale, one product).
  template <int NB>
  __device__ __forceinline__ static uint32_t bin_of(double v) {
    return (uint32_t)fmin(v, (double)(NB - 1));
  }
  template <int NB>
  __device__ __forceinline__ double vscale() const { return -((double)NB / span) / T; }
  template <int NB>
  __device__ __forceinline__ uint32_t bin(float z) const {
    return bin_of<NB>(order == 0 ? ((double)z - m) * vscale<NB>() : typ_cut(fabs((double)z - c)) * ((double)NB / span));
  }
  // The candidate test, the order key and the first-level bin of element i,
  // the typicality distance taken once; ORD is `order` (loops are compiled
  // per order).
  template <int NB, int ORD>
  __device__ __forceinline__ bool look(uint32_t bits, uint32_t i, uint64_t& K, uint32_t& b) const {
    const float z = __uint_as_float(bits);
    if constexpr (ORD == 0) {
      K = comp_key(bits, i);
      b = bin_of<NB>(((double)z - m) * vscale<NB>());
      return in(z, K) && (kT == 0 || score_key(bits, i) >= kT);
    } else {
      const double dc = typ_cut(fabs((double)z - c));
      K = score_key_of(dc, i);
      b = bin_of<NB>(dc * ((double)NB / span));
      return in(z, K) && (kT == 0 || K >= kT);
    }
  }
};

// The elements of for_each_elem, a tile at a time: fn(b, at) gets an array b
// of the lane's N element bits (N = NG * E for a whole tile, E for a short
// tile, 1 for each element of the tail) and at(q), the index of b[q].  A body
// can so issue one kind of work for every element of the tile before the next
// kind (the elements' exponentials interleave ahead of their branches).
template <typename DT, int NG, bool VEC, class Fn>
__device__ __forceinline__ void for_each_batch(const DT* __restrict__ xr, int64_t e_begin, int64_t e_end, Fn&& fn) {
  constexpr int E = Elem<DT>::E;
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  walk_groups<DT, NG, VEC>(xr, e_begin, e_full, [&](const auto& g, int64_t t0) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
    uint32_t b[NGP * E];
#pragma unroll
    for (int j = 0; j < NGP; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) b[j * E + e] = gbits<DT>(g[j], e);
    fn(b, [&](int q) { return t0 + (int64_t)(((q / E) * NT + (int)threadIdx.x) * E + q % E); });
  });
  for (int64_t i = e_full + threadIdx.x; i < e_end; i += NT) {
    const uint32_t b[1] = {gbits_at<DT>(xr, i)};
    fn(b, [&](int) { return i; });
  }
}

// Selects a loop body compiled for one order.
template <int O>
struct Ord {
  static constexpr int value = O;
};
template <class F>
__device__ __forceinline__ void by_order(int order, F&& f) {
  if (order == 0)
    f(Ord<0>{});
  else
    f(Ord<1>{});
}

// A selection in value order (order 0) with first-level bins over [0, span).
__device__ __forceinline__ NucSet value_set(double m, double thr, uint64_t kfloor, double T, const double* e2,
                                            double span = kSpan) {
  return NucSet{m, thr, kfloor, T, e2, 0, 0.0, span, 0ull};
}

// How deep a weighted selection's targets can lie, in the units of the bin
// coordinate.  Every candidate deeper than d weighs at most e^-d, and the
// heaviest candidate (depth `lead`) at least e^-lead, which bounds the total W
// from below.  With at most n candidates, those deeper than d hold less than
// n e^-d; once that is at most (1 - frac - 2 kGuard) W, the mass above d
// passes both targets of the window, (frac -+ kGuard) W.  The candidates
// deeper than the bound (plus a margin of 1 for rounding) then share the last
// guide bin, which keeps most of a peaked row out of the bins the window is
// placed in.  A bound that failed would only send the row to the one-workgroup
// fallback (its window would overflow); the selection stays exact.
__device__ __forceinline__ double crossing_depth(double frac, int64_t n, double lead) {
  const double rest = 1.0 - frac - 2.0 * kGuard;
  return rest > 0.0 ? lead + log((double)n / rest) + 1.0 : __builtin_inf();
}

// ---------------------------------------------------------------- block helpers
// last_done, and the finishing workgroup's waves then issue ahead of those of
// the streaming workgroups that share its CU (its steps are serial, theirs
// are not).
__device__ __forceinline__ bool last_of_row(SelShared& sh, uint32_t* ticket, uint32_t n) {
  if (!last_done(sh, ticket, n)) return false;
  __builtin_amdgcn_s_setprio(3);
  return true;
}


struct NucRed {
  double rd[NWAVE * 2];
  uint64_t rk[NWAVE * 2];
  uint32_t ru[NWAVE];
  uint32_t b_lo, b_hi, cnt, cnt_top;  // pick_bins results
  uint32_t n;
  uint64_t ksel;
  uint32_t bsel;
  double csel;  // walk_sorted: the cumulative mass through the chosen candidate
};

// Fixed-order sum over the workgroup (every thread gets it).
__device__ __forceinline__ double nuc_sum(NucRed& r, double v, int slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) r.rd[slot * NWAVE + wave] = v;
  __syncthreads();
  double t = r.rd[slot * NWAVE];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) t += r.rd[slot * NWAVE + q];
  return t;
}

// Exclusive prefix of one value per thread, in thread order (fixed order).
__device__ __forceinline__ double block_excl_scan_f64(NucRed& r, double v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double incl = v;
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) r.rd[wave] = incl;
  __syncthreads();
  double off = 0.0;
  for (int q = 0; q < wave; ++q) off += r.rd[q];
  return off + incl - v;
}

__device__ __forceinline__ uint32_t block_min_u32(NucRed& r, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d));
  __syncthreads();
  if (lane == 0) r.ru[wave] = v;
  __syncthreads();
  uint32_t o = r.ru[0];
  for (int q = 1; q < NWAVE; ++q) o = min(o, r.ru[q]);
  return o;
}

__device__ __forceinline__ int block_max_i32(NucRed& r, int v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) v = max(v, __shfl_xor(v, d));
  __syncthreads();
  if (lane == 0) r.ru[wave] = (uint32_t)v;
  __syncthreads();
  int o = (int)r.ru[0];
  for (int q = 1; q < NWAVE; ++q) o = max(o, (int)r.ru[q]);
  return o;
}

__device__ __forceinline__ uint32_t block_sum_u32(NucRed& r, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) v += (uint32_t)__shfl_xor((int)v, d);
  __syncthreads();
  if (lane == 0) r.ru[wave] = v;
  __syncthreads();
  uint32_t o = 0;
  for (int q = 0; q < NWAVE; ++q) o += r.ru[q];
  return o;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) { return ~wave_max_u64(~v); }

// Minimum / maximum of one float64 per thread over the workgroup (every
// thread gets it).
template <bool MAX>
__device__ __forceinline__ double block_ext_f64(NucRed& r, double v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_xor(v, d);
    v = MAX ? fmax(v, o) : fmin(v, o);
  }
  __syncthreads();
  if (lane == 0) r.rd[wave] = v;
  __syncthreads();
  double o = r.rd[0];
  for (int q = 1; q < NWAVE; ++q) o = MAX ? fmax(o, r.rd[q]) : fmin(o, r.rd[q]);
  return o;
}

// The bins [b_lo, b_hi] of nb (<= NB) whose cumulative guide mass (after
// `base`, the mass above bin 0) first reaches t0 and t1; their candidates
// (cnt) and those of bins [0, b_hi] (cnt_top).  A target past the last bin
// takes the last non-empty bin.  Each thread holds NB / NT consecutive bins;
// the thread sums are prefixed in thread order (a fixed order: within a wave
// by shuffles, then the wave totals in wave order), the thread whose prefix
// first reaches a target walks its own bins.  Six barriers.  All threads
// call; the results are in r.
template <int NB>
__device__ void pick_bins(NucRed& r, const double* hw, const uint32_t* hc, int nb, double base, double t0,
                          double t1) {
  constexpr int PT = NB / NT;
  static_assert(PT * NT == NB && (PT & (PT - 1)) == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b0 = tid * PT;
  // Neighbouring threads' bins start PT bins apart: the q-th bin of every
  // lane of a wave would lie in the same LDS banks.  Each thread reads its
  // bins from a starting point of its own instead, (q + tid) mod PT.
  auto bin_q = [&](int q) { return b0 + ((q + tid) & (PT - 1)); };
  // (every loop below issues all of its LDS reads before it uses any: bins
  // past nb read the last one and are dropped)
  __syncthreads();
  double v[PT];
  uint32_t n[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int b = min(bin_q(q), nb - 1);
    v[q] = hw[b];
    n[q] = hc[b];
  }
  double ls = 0.0;
  int lastnz = -1;
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int b = bin_q(q);
    const bool in = b < nb;
    ls += in ? v[q] : 0.0;
    if (in && n[q] != 0u) lastnz = max(lastnz, b);
  }
  double incl = ls;
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const double prev = __shfl_up(incl, 1);
  int wl = lastnz;
  for (int d = 1; d < 64; d <<= 1) wl = max(wl, __shfl_xor(wl, d));
  if (lane == 63) r.rd[wave] = incl;
  if (lane == 0) r.ru[wave] = (uint32_t)(wl + 1);
  __syncthreads();
  double excl = base;
  int last = -1;
#pragma unroll
  for (int q = 0; q < NWAVE; ++q) {
    if (q < wave) excl += r.rd[q];
    last = max(last, (int)r.ru[q] - 1);
  }
  excl = lane > 0 ? excl + prev : excl;  // this thread's cumulative mass before its bins
  const uint64_t h0 = __ballot(excl + ls >= t0), h1 = __ballot(excl + ls >= t1);
  if (lane == 0) {
    r.rk[wave] = h0 ? (uint64_t)(wave * 64 + __builtin_ctzll(h0)) : ~0ull;
    r.rk[NWAVE + wave] = h1 ? (uint64_t)(wave * 64 + __builtin_ctzll(h1)) : ~0ull;
  }
  __syncthreads();
  uint64_t f0 = ~0ull, f1 = ~0ull;
#pragma unroll
  for (int q = 0; q < NWAVE; ++q) {
    f0 = min(f0, r.rk[q]);
    f1 = min(f1, r.rk[NWAVE + q]);
  }
  // the first of the owner's bins whose cumulative mass reaches the target
  // (or its last bin, where the prefix reached it and this order's rounding
  // did not); no owner: the last non-empty bin
  auto walk = [&](double tt) {
    double w[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) w[q] = hw[min(b0 + q, nb - 1)];
    int cand = -1;
    double c = excl;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      c += b0 + q < nb ? w[q] : 0.0;
      if (cand < 0 && c >= tt) cand = b0 + q;
    }
    return (uint32_t)(cand < 0 ? min(b0 + PT - 1, nb - 1) : cand);
  };
  const uint32_t dflt = (uint32_t)(last < 0 ? 0 : last);
  if (f0 == ~0ull ? tid == 0 : (uint64_t)tid == f0) r.b_lo = f0 == ~0ull ? dflt : walk(t0);
  if (f1 == ~0ull ? tid == 0 : (uint64_t)tid == f1) r.b_hi = f1 == ~0ull ? dflt : walk(t1);
  __syncthreads();
  const int lo = (int)r.b_lo, hi = max(lo, (int)r.b_hi);
  uint32_t c = 0, ct = 0;
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int b = bin_q(q);
    if (b <= hi && b < nb) {
      ct += n[q];
      if (b >= lo) c += n[q];
    }
  }
  for (int d = 1; d < 64; d <<= 1) {
    c += (uint32_t)__shfl_xor((int)c, d);
    ct += (uint32_t)__shfl_xor((int)ct, d);
  }
  if (lane == 0) r.rk[wave] = ((uint64_t)ct << 32) | c;  // (every read of r.rk above precedes the last barrier)
  __syncthreads();
  if (tid == 0) {
    uint64_t sc = 0, st = 0;
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) {
      sc += r.rk[q] & 0xFFFFFFFFull;
      st += r.rk[q] >> 32;
    }
    r.b_hi = (uint32_t)hi;
    r.cnt = (uint32_t)min<uint64_t>(sc, 0xFFFFFFFFull);
    r.cnt_top = (uint32_t)min<uint64_t>(st, 0xFFFFFFFFull);
  }
  __syncthreads();
}

// Walk n sorted candidates (bits) with weights S.w from a cumulative mass A:
// the first index whose cumulative c satisfies c >= t (strict = false) or
// t < c (strict = true); none: the last with a positive weight (or the last).
// *cum (if given) gets the cumulative mass through the chosen candidate.  Up
// to 64 candidates: one per lane of wave 0, prefixed by shuffles; more: each
// thread sums a run of ceil(n / NT) candidates in order, the runs are
// prefixed in a fixed order, and every thread walks its own run.  All threads
// call.
template <class Bits>
__device__ uint32_t walk_sorted(NucRed& r, const Bits& bits, uint32_t n, const NucSet& S, double A, double t,
                                bool strict, double* cum = nullptr) {
  if (n <= 64) {
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const double w = (uint32_t)lane < n ? S.w(__uint_as_float(bits[lane])) : 0.0;
      double incl = w;
      for (int d = 1; d < 64; d <<= 1) {
        const double o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      const double c = A + incl;
      const bool live = (uint32_t)lane < n;
      const uint64_t hit = __ballot(live && (strict ? (t < c) : (c >= t)));
      const uint64_t pos = __ballot(live && w > 0.0);
      const int j = hit ? __builtin_ctzll(hit) : pos ? 63 - __builtin_clzll(pos) : (n > 0 ? (int)n - 1 : 0);
      const double cj = __shfl(c, j);
      if (lane == 0) {
        r.ru[0] = (uint32_t)j;
        r.csel = cj;
      }
    }
    __syncthreads();
    if (cum) *cum = r.csel;
    return r.ru[0];
  }
  const uint32_t R = (n + NT - 1) / NT;  // (<= kRun) candidates per thread
  const uint32_t j0 = threadIdx.x * R;
  double wl[kRun];
  double run = 0.0;
#pragma unroll
  for (uint32_t q = 0; q < kRun; ++q) {
    wl[q] = 0.0;
    if (q < R && j0 + q < n) wl[q] = S.w(__uint_as_float(bits[j0 + q]));
    run += wl[q];
  }
  double c = A + block_excl_scan_f64(r, run);
  uint32_t first = 0xFFFFFFFFu;
  int lastpos = -1;
  double cfirst = 0.0, clast = 0.0, cend = 0.0;
#pragma unroll
  for (uint32_t q = 0; q < kRun; ++q) {
    if (q < R && j0 + q < n) {
      c += wl[q];
      if (wl[q] > 0.0) {
        lastpos = (int)(j0 + q);
        clast = c;
      }
      if (first == 0xFFFFFFFFu && (strict ? (t < c) : (c >= t))) {
        first = j0 + q;
        cfirst = c;
      }
      if (j0 + q == n - 1) cend = c;
    }
  }
  const uint32_t f = block_min_u32(r, first);
  const int lp = block_max_i32(r, lastpos);
  const uint32_t j = f != 0xFFFFFFFFu ? f : lp >= 0 ? (uint32_t)lp : (n > 0 ? n - 1 : 0);
  if (cum) {
    // the owner of the chosen candidate's run publishes its cumulative mass
    __syncthreads();
    if (j >= j0 && j < j0 + R) r.csel = j == first ? cfirst : j == (uint32_t)lastpos ? clast : cend;
    __syncthreads();
    *cum = r.csel;
  }
  return j;
}

// ---------------------------------------------------------------- one-wave windows
// A window of up to 64 candidates, one per lane of the calling wave (lanes
// from n on hold nothing), put in (key desc) order: each lane's rank is the
// number of larger keys (keys are distinct), then the lanes trade places
// through the wave's own LDS scratch (sk, sb: 64 entries).
__device__ __forceinline__ uint64_t lane_key(uint64_t v, uint32_t j) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), (int)j) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, (int)j);
}
__device__ __forceinline__ void wave_sort(uint64_t& key, uint32_t& bits, uint32_t n, uint64_t* sk, uint32_t* sb) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t rank = 0;
  for (uint32_t j = 0; j < n; ++j) rank += lane_key(key, j) > key ? 1u : 0u;
  if (lane < n) {
    sk[rank] = key;
    sb[rank] = bits;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  key = lane < n ? sk[lane] : 0ull;
  bits = lane < n ? sb[lane] : 0u;
}
// Inclusive prefix sum over the wave in lane order (fixed order).
__device__ __forceinline__ double wave_incl_f64(double v) {
  const int lane = threadIdx.x & 63;
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}
// The first lane (< n) whose flag is set; else the last (< n) with a positive
// weight; else n - 1 (0 for none): walk_sorted's choice over one wave.
__device__ __forceinline__ uint32_t wave_pick(bool hit, bool pos, uint32_t n) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t h = __ballot(hit && lane < n), p = __ballot(pos && lane < n);
  return h ? (uint32_t)__builtin_ctzll(h) : p ? (uint32_t)(63 - __builtin_clzll(p)) : (n > 0 ? n - 1 : 0u);
}

// The window's n candidates in LDS put in (key desc) order.  Up to NT of
// them: each thread ranks its own candidate against all n (keys are distinct;
// broadcast reads) and moves it to its place through scratch past the
// window's first half; more: the bitonic network.
__device__ __forceinline__ void sort_window(uint64_t* key, uint32_t* bits, uint32_t n) {
  if (n > (uint32_t)NT) {
    sort_desc<kCapW>(key, bits, n);
    return;
  }
  const uint32_t t = threadIdx.x;
  uint64_t* sk = key + kCapW / 2;
  uint32_t* sb = bits + kCapW / 2;
  const uint64_t mine = t < n ? key[t] : 0ull;
  const uint32_t mb = t < n ? bits[t] : 0u;
  uint32_t rank = 0;
  for (uint32_t j = 0; j < n; ++j) rank += key[j] > mine ? 1u : 0u;
  if (t < n) {
    sk[rank] = mine;
    sb[rank] = mb;
  }
  __syncthreads();
  if (t < n) {
    key[t] = sk[t];
    bits[t] = sb[t];
  }
  __syncthreads();
}

// Fixed-order sum of S.w over the first n sorted candidates.
template <class Bits>
__device__ double sum_sorted(NucRed& r, const Bits& bits, uint32_t n, const NucSet& S) {
  if (n <= 64) {
    __syncthreads();
    if (threadIdx.x < 64) {
      const double v = wave_sum_f64(threadIdx.x < n ? S.w(__uint_as_float(bits[threadIdx.x])) : 0.0);
      if (threadIdx.x == 0) r.csel = v;
    }
    __syncthreads();
    return r.csel;
  }
  const uint32_t R = (n + NT - 1) / NT;  // (<= kRun) candidates per thread
  const uint32_t j0 = threadIdx.x * R;
  double run = 0.0;
  for (uint32_t q = 0; q < R; ++q)
    if (j0 + q < n) run += S.w(__uint_as_float(bits[j0 + q]));
  return nuc_sum(r, run, 0);
}

// Key range [klo, khi] split into at most kFbNB bins of 2^shift keys from the top.
__device__ __forceinline__ int key_shift(uint64_t klo, uint64_t khi) {
  const uint64_t w = khi - klo;
  const int bits = w == 0 ? 0 : 64 - __builtin_clzll(w);
  return bits > 11 ? bits - 11 : 0;
}

// ---------------------------------------------------------------- one-workgroup selection
struct FbShared {
  double hw[kFbNB];      // guide mass per bin; while sorting, the window's element bits (uint32)
  uint32_t hc[kFbNB];
  uint64_t list[kCapW];
};

struct SelOut {
  uint64_t key;   // the selected candidate
  uint32_t bits;  // its element bits
  double tot;     // the candidates' total mass (float64, fixed order)
  double cum;     // the cumulative mass through the selected candidate
};

// The weighted selection over the candidates of `S` by one workgroup alone:
// the first candidate in (value desc, id asc) order whose cumulative weight c
// satisfies c >= frac * W (strict = false) or frac * W < c (strict = true), W
// the candidates' total mass.  Guide passes narrow a window until its
// candidates fit LDS (first by steps of (m - z) / T, then by key ranges), then
// one exact pass sums the mass above it.  All threads call; all get the result.
template <typename DT, bool VEC>
__device__ SelOut wg_select(FbShared& s, NucRed& r, const DT* __restrict__ xr, int64_t V, const NucSet& S,
                            double frac, bool strict) {
  const int tid = threadIdx.x;
  __syncthreads();
  for (int b = tid; b < kFbNB; b += NT) {
    s.hw[b] = 0.0;
    s.hc[b] = 0u;
  }
  __syncthreads();
  double g = 0.0;
  for_each_elem<DT, kNG, VEC>(xr, 0, V, [&](uint32_t bits, int64_t i) {
    const float z = __uint_as_float(bits);
    if (S.in(bits, (uint32_t)i, S.key(bits, (uint32_t)i))) {
      const float gw = S.gw(z);
      const uint32_t b = S.bin<kFbNB>(z);
      __hip_atomic_fetch_add(&s.hw[b], (double)gw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_add(&s.hc[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      g += gw;
    }
  });
  __syncthreads();
  const double gtot = nuc_sum(r, g, 0);
  pick_bins<kFbNB>(r, s.hw, s.hc, kFbNB, 0.0, frac * gtot - kGuard * gtot, frac * gtot + kGuard * gtot);
  bool by_key = false;  // window by first-level bins [b_lo, b_hi], else by keys [klo, khi]
  const uint32_t b_lo = r.b_lo, b_hi = r.b_hi;
  uint64_t klo = 0, khi = 0;
  double tot = 0.0, A = 0.0;
  uint32_t* lbits = reinterpret_cast<uint32_t*>(s.hw);
  for (int level = 0;; ++level) {
    // exact pass: the total and the mass above the window in float64 (fixed
    // order), the window's candidates into LDS, the window's key range
    __syncthreads();
    if (tid == 0) r.n = 0u;
    __syncthreads();
    double t_l = 0.0, a_l = 0.0;
    uint64_t kmin = ~0ull, kmax = 0ull;
    for_each_elem<DT, kNG, VEC>(xr, 0, V, [&](uint32_t bits, int64_t i) {
      const float z = __uint_as_float(bits);
      const uint64_t K = S.key(bits, (uint32_t)i);
      if (!S.in(bits, (uint32_t)i, K)) return;
      const double w = S.w(z);
      t_l += w;
      bool above, inw;
      if (by_key) {
        above = K > khi;
        inw = !above && K >= klo;
      } else {
        const uint32_t b = S.bin<kFbNB>(z);
        above = b < b_lo;
        inw = !above && b <= b_hi;
      }
      if (above) a_l += w;
      if (inw) {
        kmin = min(kmin, K);
        kmax = max(kmax, K);
        const uint32_t p = atomicAdd(&r.n, 1u);
        if (p < kCapW) {
          s.list[p] = K;
          lbits[p] = bits;
        }
      }
    });
    tot = nuc_sum(r, t_l, 0);
    A = nuc_sum(r, a_l, 1);
    {
      const int lane = tid & 63, wave = tid >> 6;
      kmin = wave_min_u64(kmin);
      kmax = wave_max_u64(kmax);
      if (lane == 0) {
        r.rk[wave] = kmin;
        r.rk[NWAVE + wave] = kmax;
      }
      __syncthreads();
      kmin = r.rk[0];
      kmax = r.rk[NWAVE];
#pragma unroll
      for (int q = 1; q < NWAVE; ++q) {
        kmin = min(kmin, r.rk[q]);
        kmax = max(kmax, r.rk[NWAVE + q]);
      }
    }
    if (r.n <= kCapW || level == kMaxLevels) break;
    // too many: narrow the window by a guide pass over its key range
    klo = kmin;
    khi = kmax;
    by_key = true;
    const int sh = key_shift(klo, khi);
    __syncthreads();
    for (int b = tid; b < kFbNB; b += NT) {
      s.hw[b] = 0.0;
      s.hc[b] = 0u;
    }
    __syncthreads();
    for_each_elem<DT, kNG, VEC>(xr, 0, V, [&](uint32_t bits, int64_t i) {
      const float z = __uint_as_float(bits);
      const uint64_t K = S.key(bits, (uint32_t)i);
      if (!S.in(bits, (uint32_t)i, K) || K > khi || K < klo) return;
      const uint32_t b = (uint32_t)((khi - K) >> sh);
      __hip_atomic_fetch_add(&s.hw[b], (double)S.gw(z), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_add(&s.hc[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    });
    __syncthreads();
    const int nb = (int)((khi - klo) >> sh) + 1;
    pick_bins<kFbNB>(r, s.hw, s.hc, nb, A, frac * tot - kGuard * tot, frac * tot + kGuard * tot);
    // the chosen bins as a key range
    const uint64_t c_lo = r.b_lo, c_hi = r.b_hi;
    const uint64_t top = c_lo << sh;                         // offset of the window's top below khi
    const uint64_t bot = (c_hi << sh) + ((1ull << sh) - 1);  // offset of its lowest key (may pass klo)
    const uint64_t khi2 = khi - top;
    klo = (bot >= khi - klo) ? klo : khi - bot;
    khi = khi2;
  }
  const uint32_t n = min(r.n, kCapW);
  sort_desc<kCapW>(s.list, lbits, n);
  double cum = 0.0;
  const uint32_t j = walk_sorted(r, lbits, n, S, A, frac * tot, strict, &cum);
  if (tid == 0) {
    r.ksel = s.list[j];
    r.bsel = lbits[j];
  }
  __syncthreads();
  const SelOut o{r.ksel, r.bsel, tot, cum};
  __syncthreads();
  return o;
}

// Smallest composite key of an element with value >= thr.  (Keys of
// consecutive floats differ by one, so the next float up is key + 1.)
__device__ __forceinline__ uint64_t key_floor(double thr) {
  const float v = (float)thr;
  uint32_t k = fkey(__float_as_uint(v));
  if ((double)v < thr) k += 1u;
  return (uint64_t)k << 32;
}

// ---------------------------------------------------------------- the parallel passes
struct NucCommon {
  int64_t e_begin, e_end;
  double m, thr;
  uint64_t kmp;  // smallest key min_p keeps (0: min_p off)
  double span1;  // the cut's guide bins (untempered, value order) cover [0, span1)
};

__device__ __forceinline__ NucCommon nuc_common(const NucArgs& a, int64_t row, int seg) {
  NucCommon c;
  c.e_begin = (int64_t)seg * a.seg_len;
  c.e_end = min(a.V, c.e_begin + a.seg_len);
  c.m = a.st_max[row];
  c.thr = a.top_n_sigma > 0.0f ? c.m - (double)a.top_n_sigma * a.sigma[row] : -__builtin_inf();
  c.kmp = a.min_p > 0.0f ? key_floor(c.m + log((double)a.min_p)) : 0ull;
  c.span1 = fmin(kSpan, crossing_depth((double)a.top_p, a.V, 0.0));
  return c;
}

// The whole row by one workgroup: the cut, min_p, the draw.
template <typename DT, bool VEC>
__device__ void row_alone(FbShared& s, NucRed& r, const NucArgs& a, int64_t row, const NucCommon& c,
                          const DT* __restrict__ xr, const double* e2) {
  const NucSet S1 = value_set(c.m, c.thr, 0ull, 1.0, e2, c.span1);
  const SelOut cut = wg_select<DT, VEC>(s, r, xr, a.V, S1, (double)a.top_p, false);
  const uint64_t kfin = max(cut.key, c.kmp);
  const NucSet S2 = value_set(c.m, c.thr, kfin, (double)a.T, e2);
  // floor mode: only the kept set's total (a selection at 0 returns it)
  const SelOut d = wg_select<DT, VEC>(s, r, xr, a.V, S2, a.out_kfl ? 0.0 : (double)a.u[row], true);
  if (threadIdx.x == 0) {
    if (a.out_kfl) {
      a.out_kfl[row] = kfin;
      a.out_lse_f[row] = c.m / (double)a.T + log(d.tot);
      return;
    }
    a.out_token[row] = ~(uint32_t)d.key;
    if (a.out_logp) a.out_logp[row] = (float)(((double)__uint_as_float(d.bits) - c.m) / (double)a.T - log(d.tot));
  }
}

// The last guide bin's mass and count, kept per lane while streaming (most
// elements of a peaked row land there), added with one LDS atomic per wave.
__device__ __forceinline__ void add_deep(double* hw, uint32_t* hc, double w, uint32_t n) {
  w = wave_sum_f64(w);
  for (int d = 1; d < 64; d <<= 1) n += (uint32_t)__shfl_xor((int)n, d);
  if ((threadIdx.x & 63) == 0 && n != 0u) {
    __hip_atomic_fetch_add(&hw[kNB - 1], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(&hc[kNB - 1], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// LDS histogram -> the row's global histogram (device-scope atomics,
// complete when the workgroup arrives at its ticket).  The highest non-empty
// bin short of the last goes to *top (an atomic max per wave), so that the
// row's last workgroup clears only the bins up to it.
__device__ __forceinline__ void flush_hist(const double* hw, const uint32_t* hc, double* gw, uint32_t* gc,
                                           uint32_t* top) {
  constexpr int Q = kNB / NT;
  uint32_t c[Q];
  double w[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {  // (all LDS reads first)
    c[q] = hc[q * NT + threadIdx.x];
    w[q] = hw[q * NT + threadIdx.x];
  }
  int hi = -1;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int b = q * NT + (int)threadIdx.x;
    if (c[q]) {
      (void)__hip_atomic_fetch_add(&gw[b], w[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      (void)__hip_atomic_fetch_add(&gc[b], c[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (b < kNB - 1) hi = b;
    }
  }
  for (int d = 1; d < 64; d <<= 1) hi = max(hi, __shfl_xor(hi, d));
  if ((threadIdx.x & 63) == 0 && hi >= 0)
    (void)__hip_atomic_fetch_max(top, (uint32_t)hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The row's global histogram -> LDS.  Each thread issues all of its loads
// before it waits for any.  (clear_hist zeroes it afterwards.)
__device__ __forceinline__ void take_hist(double* hw, uint32_t* hc, const double* gw, const uint32_t* gc) {
  constexpr int Q = kNB / NT;
  __syncthreads();
  double v[Q];
  uint32_t c[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    v[q] = ld_dev(&gw[q * NT + threadIdx.x]);
    c[q] = ld_dev(&gc[q * NT + threadIdx.x]);
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int b = q * NT + threadIdx.x;
    hw[b] = v[q];
    hc[b] = c[q];
  }
  __syncthreads();
}

// The same in two halves, so that a tail can issue these loads together with
// others: load_hist into registers, put_hist into LDS (then a barrier).
constexpr int kHQ = kNB / NT;
__device__ __forceinline__ void load_hist(const double* gw, const uint32_t* gc, double (&v)[kHQ],
                                          uint32_t (&c)[kHQ]) {
#pragma unroll
  for (int q = 0; q < kHQ; ++q) {
    v[q] = ld_dev(&gw[q * NT + threadIdx.x]);
    c[q] = ld_dev(&gc[q * NT + threadIdx.x]);
  }
}
__device__ __forceinline__ void put_hist(double* hw, uint32_t* hc, const double (&v)[kHQ], const uint32_t (&c)[kHQ]) {
#pragma unroll
  for (int q = 0; q < kHQ; ++q) {
    hw[q * NT + threadIdx.x] = v[q];
    hc[q * NT + threadIdx.x] = c[q];
  }
  __syncthreads();
}

// The row's n (<= kCapW) window candidates -> LDS, all loads issued first;
// (k0, b0) is this thread's first candidate, loaded earlier (before n was
// known, together with the tail's other loads).
__device__ __forceinline__ void take_list_pf(uint64_t* key, uint32_t* bits, const uint64_t* lkey,
                                             const uint32_t* lbits, uint32_t n, uint64_t k0, uint32_t b0) {
  constexpr int Q = kCapW / NT;
  uint64_t k[Q];
  uint32_t b[Q];
#pragma unroll
  for (int q = 1; q < Q; ++q) {
    const uint32_t j = q * NT + threadIdx.x;
    if (j < n) {
      k[q] = ld_dev(&lkey[j]);
      b[q] = ld_dev(&lbits[j]);
    }
  }
  if (threadIdx.x < n) {
    key[threadIdx.x] = k0;
    bits[threadIdx.x] = b0;
  }
#pragma unroll
  for (int q = 1; q < Q; ++q) {
    const uint32_t j = q * NT + threadIdx.x;
    if (j < n) {
      key[j] = k[q];
      bits[j] = b[q];
    }
  }
  __syncthreads();
}

// The row's n (<= kCapW) window candidates -> LDS, all loads issued first.
__device__ __forceinline__ void take_list(uint64_t* key, uint32_t* bits, const uint64_t* lkey, const uint32_t* lbits,
                                          uint32_t n) {
  constexpr int Q = kCapW / NT;
  uint64_t k[Q];
  uint32_t b[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint32_t j = q * NT + threadIdx.x;
    if (j < n) {
      k[q] = ld_dev(&lkey[j]);
      b[q] = ld_dev(&lbits[j]);
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint32_t j = q * NT + threadIdx.x;
    if (j < n) {
      key[j] = k[q];
      bits[j] = b[q];
    }
  }
  __syncthreads();
}

// The row's global histogram back to zero: the bins up to *top and the last
// (no others were written), and *top itself.  Called where no barrier
// follows, so no wave waits for these stores.
__device__ __forceinline__ void clear_hist(double* gw, uint32_t* gc, uint32_t* top) {
  const uint32_t t = ld_dev(top);
  for (uint32_t b = threadIdx.x; b <= t; b += NT) {
    st_dev(&gw[b], 0.0);
    st_dev(&gc[b], 0u);
  }
  if (threadIdx.x == 0) {
    st_dev(&gw[kNB - 1], 0.0);
    st_dev(&gc[kNB - 1], 0u);
    st_dev(top, 0u);
  }
}

// Window candidates of one workgroup: staged in LDS as indices within the
// segment while streaming, then given positions in the row's list with one
// counter atomic and written out (their values re-read from the cache).
// Past the list's end they are only counted.
struct Stage {
  uint32_t idx[kCapW];
  uint32_t n;
  uint32_t base;
};

__device__ __forceinline__ void stage_window(Stage& st, int64_t i, int64_t e_begin) {
  const uint32_t p = atomicAdd(&st.n, 1u);
  if (p < kCapW) st.idx[p] = (uint32_t)(i - e_begin);
}

template <typename DT>
__device__ __forceinline__ void flush_window(Stage& st, const DT* __restrict__ xr, int64_t e_begin, uint32_t* cnt,
                                             uint64_t* lkey, uint32_t* lbits, const NucSet* order = nullptr) {
  __syncthreads();
  const uint32_t n = st.n;
  if (n == 0) return;
  if (threadIdx.x == 0) st.base = __hip_atomic_fetch_add(cnt, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t base = st.base;
  for (uint32_t j = threadIdx.x; j < min(n, kCapW); j += NT) {
    const uint32_t pos = base + j;
    if (pos < kCapW) {
      const int64_t i = e_begin + st.idx[j];
      const uint32_t bits = gbits_at<DT>(xr, i);
      st_dev(&lkey[pos], order ? order->key(bits, (uint32_t)i) : comp_key(bits, (uint32_t)i));
      st_dev(&lbits[pos], bits);
    }
  }
}

// The candidates a first guide pass gathers (those within the crossing
// bound): staged without atomics, each wave in a region of its own, placed by
// a ballot and the lanes' ranks (the wave's count is a uniform register); past
// a region's end they are only counted.  Their bits are staged with them, so
// the flush reads nothing back from the row.
struct GatherStage {
  static constexpr uint32_t kPer = kGatherCap / NWAVE;
  uint32_t idx[NWAVE][kPer];
  uint32_t bits[NWAVE][kPer];
  uint32_t n[NWAVE];
};

__device__ __forceinline__ void gather(GatherStage& st, uint32_t& cnt, bool take, int64_t i, int64_t e_begin,
                                       uint32_t bits) {
  if (cnt > GatherStage::kPer) return;  // the region overflowed: its count stays past the end
  const uint64_t m = __ballot(take);
  if (m != 0ull) {
    const uint32_t p = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (take && p < GatherStage::kPer) {
      st.idx[threadIdx.x >> 6][p] = (uint32_t)(i - e_begin);
      st.bits[threadIdx.x >> 6][p] = bits;
    }
    cnt += (uint32_t)__builtin_popcountll(m);
  }
}

// The workgroup's gathered candidates -> its (row, segment) slot, wave after
// wave in stream order (a fixed order), with the count (kGatherCap + 1 when
// a wave's region overflowed; the slot is then left unwritten).  All threads
// call, each wave with its count.
__device__ __forceinline__ void flush_gather(GatherStage& st, uint32_t cnt, int64_t e_begin, const NucArgs& a,
                                             int64_t row, int seg) {
  if ((threadIdx.x & 63) == 0) st.n[threadIdx.x >> 6] = cnt;
  __syncthreads();
  uint32_t off[NWAVE], tot = 0;
  bool over = false;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    off[w] = tot;
    tot += min(st.n[w], GatherStage::kPer);
    over = over || st.n[w] > GatherStage::kPer;
  }
  const size_t slot = (size_t)(row * a.S + seg);
  if (threadIdx.x == 0) st_dev(&a.gcnt[slot], over ? (uint32_t)kGatherCap + 1u : tot);
  if (over) return;
  uint32_t* gb = a.gbits + slot * kGatherCap;
  uint32_t* gi = a.gidx + slot * kGatherCap;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    const uint32_t nw = min(st.n[w], GatherStage::kPer);
    for (uint32_t j = threadIdx.x; j < nw; j += NT) {
      gb[off[w] + j] = st.bits[w][j];
      gi[off[w] + j] = (uint32_t)(e_begin + st.idx[w][j]);
    }
  }
}

// The elements a pass visits in its (row, segment): the segment itself, or,
// for a row whose gathered list holds every candidate the pass can reach, the
// candidates gathered from that segment (fn gets each one's bits and index).
template <typename DT, bool VEC, class Fn>
__device__ __forceinline__ void for_each_cand(const NucArgs& a, int64_t row, int seg, bool listed,
                                              const DT* __restrict__ xr, int64_t e_begin, int64_t e_end, Fn&& fn) {
  if (listed) {
    const size_t slot = (size_t)(row * a.S + seg);
    const uint32_t n = min(a.gcnt[slot], (uint32_t)kGatherCap);
    const uint32_t* gb = a.gbits + slot * kGatherCap;
    const uint32_t* gi = a.gidx + slot * kGatherCap;
    for (uint32_t j = threadIdx.x; j < n; j += NT) fn(gb[j], (int64_t)gi[j]);
    return;
  }
  for_each_elem<DT, kNG, VEC>(xr, e_begin, e_end, fn);
}

// for_each_cand a tile at a time, as for_each_batch (a gathered list one
// candidate at a time).
template <typename DT, bool VEC, class Fn>
__device__ __forceinline__ void for_each_cand_batch(const NucArgs& a, int64_t row, int seg, bool listed,
                                                    const DT* __restrict__ xr, int64_t e_begin, int64_t e_end,
                                                    Fn&& fn) {
  if (listed) {
    const size_t slot = (size_t)(row * a.S + seg);
    const uint32_t n = min(a.gcnt[slot], (uint32_t)kGatherCap);
    const uint32_t* gb = a.gbits + slot * kGatherCap;
    const uint32_t* gi = a.gidx + slot * kGatherCap;
    for (uint32_t j = threadIdx.x; j < n; j += NT) {
      const uint32_t b[1] = {gb[j]};
      const int64_t i = (int64_t)gi[j];
      fn(b, [&](int) { return i; });
    }
    return;
  }
  for_each_batch<DT, kNG, VEC>(xr, e_begin, e_end, fn);
}

union NucLds {
  struct {
    double hw[kNB];
    uint32_t hc[kNB];
  } h;
  struct {
    uint64_t key[kCapW];
    uint32_t bits[kCapW];
  } w;
};

// A pass that stages window candidates while it streams and sorts the row's
// window only afterwards, in the row's last workgroup, keeps both in the
// same LDS.
union StageOrWindow {
  NucLds L;
  Stage st;
};

// Pass 1: guide histogram of exp(z - m) over the candidates and their exact
// total, and the candidates within the crossing bound (the bins short of the
// last) gathered per segment; the last workgroup places the cut window.  When
// every segment's gathered candidates fit and the window stays short of the
// last bin, the later passes visit only the gathered candidates.
template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void nuc_hist_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ NucLds L;
  __shared__ GatherStage gs;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  if (a.st_bad[row]) {
    if (seg == 0 && tid == 0) {
      if (a.out_kfl) {  // (the caller fails such rows closed)
        a.out_kfl[row] = 0ull;
        a.out_lse_f[row] = __builtin_nan("");
      } else {
        a.out_token[row] = kFail;
        if (a.out_logp) a.out_logp[row] = __builtin_nanf("");
      }
    }
    return;
  }
  init_e2(e2);
  const NucCommon c = nuc_common(a, row, seg);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  const NucSet S1 = value_set(c.m, c.thr, 0ull, 1.0, e2, c.span1);
  for (int b = tid; b < kNB; b += NT) {
    L.h.hw[b] = 0.0;
    L.h.hc[b] = 0u;
  }
  __syncthreads();
  double z0 = 0.0;
  uint32_t dn = 0, ng = 0;
  for_each_batch<DT, kNG, VEC>(xr, c.e_begin, c.e_end, [&](const auto& bits, auto at) {
    constexpr int N = (int)(sizeof(bits) / sizeof(bits[0]));
    // the exact weights first, every element's (free of branches, so that
    // the tile's exponentials interleave); they serve the guide too
    double w[N];
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const float z = __uint_as_float(bits[q]);
      w[q] = S1.w_if(z > -__builtin_inff() && (double)z >= c.thr, z);
    }
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const float z = __uint_as_float(bits[q]);
      const bool ok = z > -__builtin_inff() && (double)z >= c.thr;
      const uint32_t b = S1.bin<kNB>(z);
      const bool shallow = ok && b < kNB - 1;
      if (shallow) {
        __hip_atomic_fetch_add(&L.h.hw[b], w[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&L.h.hc[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      gather(gs, ng, shallow, at(q), c.e_begin, bits[q]);
      dn += ok && b == kNB - 1 ? 1u : 0u;
      z0 += w[q];
    }
  });
  // The last bin gets the deep candidates' count but not their mass: a target
  // past the other bins' mass falls to the last non-empty bin, which is the
  // last bin whenever it holds candidates, as it would with the mass.
  add_deep(L.h.hw, L.h.hc, 0.0, dn);
  flush_gather(gs, ng, c.e_begin, a, row, seg);
  __syncthreads();
  double* gw = a.h0w + row * kNB;
  uint32_t* gc = a.h0c + row * kNB;
  flush_hist(L.h.hw, L.h.hc, gw, gc, &a.plan[row].h0top);
  z0 = nuc_sum(r, z0, 0);
  if (tid == 0) st_dev(&a.p_z0[row * a.S + seg], z0);
  if (!last_of_row(sh, a.tickets + row * 3, (uint32_t)a.S)) return;
  // ---- the row's last workgroup: its global loads issued together
  const int64_t p0 = row * a.S;
  const double vz = tid < a.S ? ld_dev(&a.p_z0[p0 + tid]) : 0.0;
  const int vg = tid < a.S ? (int)ld_dev(&a.gcnt[p0 + tid]) : 0;
  double hv[kHQ];
  uint32_t hcv[kHQ];
  load_hist(gw, gc, hv, hcv);
  const double Z0 = block_sum_f64(sh, vz);
  const bool fit = block_max_i32(r, vg) <= kGatherCap;
  put_hist(L.h.hw, L.h.hc, hv, hcv);
  const double t = (double)a.top_p * Z0, g = kGuard * Z0;
  pick_bins<kNB>(r, L.h.hw, L.h.hc, kNB, 0.0, t - g, t + g);
  const bool listed = fit && r.b_hi < (uint32_t)kNB - 1;
  const uint32_t b_lo = r.cnt_top <= kCapW ? 0u : r.b_lo;  // from the top of the row when it fits
  // The exact mass above the window: the bins above it hold the exact weights
  // of their candidates (summed in the order the atomics landed, like the
  // guide that placed the window), taken here in bin order.
  double av = 0.0;
#pragma unroll
  for (int q = 0; q < kNB / NT; ++q) {
    const uint32_t b = (uint32_t)tid * (kNB / NT) + q;
    av += b < b_lo ? L.h.hw[b] : 0.0;
  }
  const double above = nuc_sum(r, av, 0);
  if (tid == 0) {
    NucPlan& p = a.plan[row];
    p.b_lo = b_lo;
    p.b_hi = r.b_hi;
    p.z0 = Z0;
    p.a_above = above;
    p.listed = listed ? 1u : 0u;
    p.state = 0u;
  }
  clear_hist(gw, gc, &a.plan[row].h0top);
}

// Pass 2: the exact mass above the cut window and the window's candidates; the
// tempered guide histogram and exact mass of the kept candidates above it.
// The last workgroup cuts, applies min_p and draws, or places the draw window.
template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void nuc_collect_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ NucLds L;
  __shared__ Stage st;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows || a.st_bad[row]) return;
  if (tid == 0) st.n = 0u;
  init_e2(e2);
  const NucCommon c = nuc_common(a, row, seg);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  const uint32_t b_lo = a.plan[row].b_lo, b_hi = a.plan[row].b_hi;
  const double z0 = a.plan[row].z0;
  const NucSet S1 = value_set(c.m, c.thr, 0ull, 1.0, e2, c.span1);
  const NucSet ST = value_set(c.m, c.thr, c.kmp, (double)a.T, e2);
  for (int b = tid; b < kNB; b += NT) {
    L.h.hw[b] = 0.0;
    L.h.hc[b] = 0u;
  }
  __syncthreads();
  uint64_t* lkey = a.lkey + row * kCapW;
  uint32_t* lbits = a.lbits + row * kCapW;
  // The exact mass above the window comes from the guide pass.  The kept
  // candidates above it need their tempered weights here only for the draw's
  // guide, at T != 1 or with min_p; otherwise their mass is that one.
  const bool same_t = a.T == 1.0f, want_guide = a.out_kfl == nullptr;
  const bool need_wt = want_guide || !same_t || c.kmp != 0ull;
  double AT = 0.0;
  // A tile's bins first; a tile with a kept candidate above the window
  // anywhere in the wave takes the tempered weights of all its elements at
  // once (0 for the others, free of branches so that they interleave), a tile
  // without one none.
  for_each_cand_batch<DT, VEC>(a, row, seg, a.plan[row].listed != 0u, xr, c.e_begin, c.e_end,
                               [&](const auto& bits, auto at) {
    constexpr int N = (int)(sizeof(bits) / sizeof(bits[0]));
    uint32_t b[N];
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const float z = __uint_as_float(bits[q]);
      const bool cand = z > -__builtin_inff() && (double)z >= c.thr;
      b[q] = cand ? S1.bin<kNB>(z) : (uint32_t)kNB;
    }
    if (need_wt) {
      bool kept[N], any = false;
#pragma unroll
      for (int q = 0; q < N; ++q) {
        kept[q] = b[q] < b_lo && comp_key(bits[q], (uint32_t)at(q)) >= c.kmp;
        any = any || kept[q];
      }
      if (__ballot(any) != 0ull) {
        double wt[N];
#pragma unroll
        for (int q = 0; q < N; ++q) wt[q] = ST.w_if(kept[q], __uint_as_float(bits[q]));
#pragma unroll
        for (int q = 0; q < N; ++q) {
          AT += wt[q];
          if (want_guide && kept[q]) {
            const uint32_t bt = ST.bin<kNB>(__uint_as_float(bits[q]));  // (its own span, also at T = 1)
            __hip_atomic_fetch_add(&L.h.hw[bt], wt[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(&L.h.hc[bt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (b[q] >= b_lo && b[q] <= b_hi) stage_window(st, at(q), c.e_begin);
  });
  flush_window<DT>(st, xr, c.e_begin, &a.lcnt[row], lkey, lbits);
  __syncthreads();
  double* gw = a.hTw + row * kNB;
  uint32_t* gc = a.hTc + row * kNB;
  uint32_t* htop = &a.plan[row].hTtop;
  flush_hist(L.h.hw, L.h.hc, gw, gc, htop);
  if (need_wt) {
    AT = nuc_sum(r, AT, 1);
    if (tid == 0) st_dev(&a.p_at[row * a.S + seg], AT);
  }
  if (!last_of_row(sh, a.tickets + row * 3 + 1, (uint32_t)a.S)) return;
  // ---- the row's last workgroup: its first global loads issued together
  const int64_t p0 = row * a.S;
  const double vat = need_wt && tid < a.S ? ld_dev(&a.p_at[p0 + tid]) : 0.0;
  const uint32_t n = ld_dev(&a.lcnt[row]);
  const uint64_t k0 = ld_dev(&lkey[tid]);
  const uint32_t b0 = ld_dev(&lbits[tid]);
  const double Atot = a.plan[row].a_above;
  const double ATtot = need_wt ? block_sum_f64(sh, vat) : Atot;
  if (tid == 0) st_dev(&a.lcnt[row], 0u);
  if (n > kCapW) {
    // the window is too crowded for LDS: the row is left to nuc_alone
    if (tid == 0) a.plan[row].state = 3u;
    clear_hist(gw, gc, htop);
    return;
  }
  const double tcut = (double)a.top_p * z0;
  uint64_t kfin;
  double WT;
  if (n <= 64) {
    // a small window: the cut, min_p and the draw by wave 0 alone, the window
    // in its lanes (no barriers); the others wait for the outcome
    if (tid < 64) {
      uint64_t key = (uint32_t)tid < n ? k0 : 0ull;
      uint32_t bits = (uint32_t)tid < n ? b0 : 0u;
      wave_sort(key, bits, n, L.w.key, L.w.bits);
      const bool live = (uint32_t)tid < n;
      const double w1 = live ? S1.w(__uint_as_float(bits)) : 0.0;
      const uint32_t jc = wave_pick(Atot + wave_incl_f64(w1) >= tcut, w1 > 0.0, n);
      const uint64_t kf = max(lane_key(key, jc), c.kmp);
      const uint32_t nk = (uint32_t)__builtin_popcountll(__ballot(live && key >= kf));
      const NucSet S2 = value_set(c.m, c.thr, kf, (double)a.T, e2);
      const double w2 = (uint32_t)tid < nk ? S2.w(__uint_as_float(bits)) : 0.0;
      const double wt = ATtot + wave_sum_f64(w2);
      uint32_t above = 0u;
      if (a.out_kfl) {  // floor mode: the kept set, nothing drawn
        if (tid == 0) {
          a.out_kfl[row] = kf;
          a.out_lse_f[row] = c.m / (double)a.T + log(wt);
          a.plan[row].state = 2u;
        }
      } else {
        const double t2 = (double)a.u[row] * wt;
        if (t2 < ATtot) {
          above = 1u;
        } else {
          const uint32_t jd = wave_pick(t2 < ATtot + wave_incl_f64(w2), w2 > 0.0, nk);
          if ((uint32_t)tid == jd) {
            a.out_token[row] = ~(uint32_t)key;
            if (a.out_logp)
              a.out_logp[row] = (float)(((double)__uint_as_float(bits) - c.m) / (double)a.T - log(wt));
            a.plan[row].state = 2u;
          }
        }
      }
      if (tid == 0) {
        r.ru[0] = above;
        r.ksel = kf;
        r.csel = wt;
      }
    }
    __syncthreads();
    if (r.ru[0] == 0u) {
      clear_hist(gw, gc, htop);
      return;
    }
    kfin = r.ksel;
    WT = r.csel;
  } else {
    take_list_pf(L.w.key, L.w.bits, lkey, lbits, n, k0, b0);
    sort_window(L.w.key, L.w.bits, n);
    // the cut, then min_p: the kept candidates of the window are its first nk
    const uint32_t jc = walk_sorted(r, L.w.bits, n, S1, Atot, tcut, false);
    kfin = max(L.w.key[jc], c.kmp);
    uint32_t nk = 0;
    for (uint32_t j = tid; j < n; j += NT) nk += L.w.key[j] >= kfin ? 1u : 0u;
    nk = block_sum_u32(r, nk);
    const NucSet S2 = value_set(c.m, c.thr, kfin, (double)a.T, e2);
    WT = ATtot + sum_sorted(r, L.w.bits, nk, S2);
    if (a.out_kfl) {  // floor mode: the kept set, nothing drawn
      if (tid == 0) {
        a.out_kfl[row] = kfin;
        a.out_lse_f[row] = c.m / (double)a.T + log(WT);
        a.plan[row].state = 2u;
      }
      clear_hist(gw, gc, htop);
      return;
    }
    const double t2 = (double)a.u[row] * WT;
    if (t2 >= ATtot) {
      const uint32_t jd = walk_sorted(r, L.w.bits, nk, S2, ATtot, t2, true);
      if (tid == 0) {
        a.out_token[row] = ~(uint32_t)L.w.key[jd];
        if (a.out_logp)
          a.out_logp[row] = (float)(((double)__uint_as_float(L.w.bits[jd]) - c.m) / (double)a.T - log(WT));
        a.plan[row].state = 2u;
      }
      clear_hist(gw, gc, htop);
      return;
    }
  }
  {
    // the draw falls above the window: place the draw window
    const double t2 = (double)a.u[row] * WT;
    take_hist(L.h.hw, L.h.hc, gw, gc);
    pick_bins<kNB>(r, L.h.hw, L.h.hc, kNB, 0.0, t2 - kGuard * WT, t2 + kGuard * WT);
    if (tid == 0) {
      NucPlan& q = a.plan[row];
      q.c_lo = r.b_lo;
      q.c_hi = r.b_hi;
      q.wt = WT;
      q.kfin = kfin;
      q.state = 1u;
    }
    clear_hist(gw, gc, htop);
  }
}

// Pass 2 in floor mode (the kept set of filtered speculative acceptance, no
// draw): nothing needs the tempered guide, so the workgroup's LDS is the
// window's staging while the segment streams and the row's window keys in
// the row's last workgroup, one union of 32 KB (four workgroups per CU where
// the drawing pass fits two).  A window candidate's key gives back its
// weight (+0 and -0, which keys fold together, weigh the same), so the
// window is sorted as keys alone.  Same decisions, in the same order, as
// nuc_collect_kernel's floor mode.
struct KeyBits {
  const uint64_t* k;
  __device__ __forceinline__ uint32_t operator[](uint32_t j) const { return key_bits((uint32_t)(k[j] >> 32)); }
};
union FloorLds {
  Stage st;
  uint64_t key[kCapW];
};

// key[0..n) (distinct keys, n <= kCapW) put in descending order: ranks
// through scratch past the first half for up to NT keys, else the bitonic
// network (zero padding, never above a real key).
__device__ __forceinline__ void sort_keys_desc(uint64_t* key, uint32_t n) {
  const uint32_t t = threadIdx.x;
  if (n <= (uint32_t)NT) {
    uint64_t* sk = key + kCapW / 2;
    const uint64_t mine = t < n ? key[t] : 0ull;
    uint32_t rank = 0;
    for (uint32_t j = 0; j < n; ++j) rank += key[j] > mine ? 1u : 0u;
    if (t < n) sk[rank] = mine;
    __syncthreads();
    if (t < n) key[t] = sk[t];
    __syncthreads();
    return;
  }
  uint32_t P = 1;
  while (P < n) P <<= 1;
  for (uint32_t i = n + t; i < P; i += NT) key[i] = 0ull;
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (uint32_t i = t; i < P / 2; i += NT) {
        const uint32_t lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        const uint64_t x = key[lo], y = key[hi];
        if ((lo & size) == 0 ? (x < y) : (x > y)) {
          key[lo] = y;
          key[hi] = x;
        }
      }
    }
  }
  __syncthreads();
}

template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void nuc_collect_floor_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ FloorLds F;
  __shared__ uint32_t s_bits[64];
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows || a.st_bad[row]) return;
  if (tid == 0) F.st.n = 0u;
  init_e2(e2);
  const NucCommon c = nuc_common(a, row, seg);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  const uint32_t b_lo = a.plan[row].b_lo, b_hi = a.plan[row].b_hi;
  const double z0 = a.plan[row].z0;
  const NucSet S1 = value_set(c.m, c.thr, 0ull, 1.0, e2, c.span1);
  const NucSet ST = value_set(c.m, c.thr, c.kmp, (double)a.T, e2);
  uint64_t* lkey = a.lkey + row * kCapW;
  uint32_t* lbits = a.lbits + row * kCapW;
  // The kept mass above the window: the guide pass's exact mass at T = 1
  // without min_p, else the tempered weights of the kept candidates there.
  const bool need_wt = a.T != 1.0f || c.kmp != 0ull;
  double AT = 0.0;
  for_each_cand_batch<DT, VEC>(a, row, seg, a.plan[row].listed != 0u, xr, c.e_begin, c.e_end,
                               [&](const auto& bits, auto at) {
    constexpr int N = (int)(sizeof(bits) / sizeof(bits[0]));
    uint32_t b[N];
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const float z = __uint_as_float(bits[q]);
      const bool cand = z > -__builtin_inff() && (double)z >= c.thr;
      b[q] = cand ? S1.bin<kNB>(z) : (uint32_t)kNB;
    }
    if (need_wt) {
      bool kept[N], any = false;
#pragma unroll
      for (int q = 0; q < N; ++q) {
        kept[q] = b[q] < b_lo && comp_key(bits[q], (uint32_t)at(q)) >= c.kmp;
        any = any || kept[q];
      }
      if (__ballot(any) != 0ull) {
#pragma unroll
        for (int q = 0; q < N; ++q) AT += ST.w_if(kept[q], __uint_as_float(bits[q]));
      }
    }
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (b[q] >= b_lo && b[q] <= b_hi) stage_window(F.st, at(q), c.e_begin);
  });
  flush_window<DT>(F.st, xr, c.e_begin, &a.lcnt[row], lkey, lbits);
  if (need_wt) {
    AT = nuc_sum(r, AT, 1);
    if (tid == 0) st_dev(&a.p_at[row * a.S + seg], AT);
  }
  if (!last_of_row(sh, a.tickets + row * 3 + 1, (uint32_t)a.S)) return;
  // ---- the row's last workgroup: its first global loads issued together
  const int64_t p0 = row * a.S;
  const double vat = need_wt && tid < a.S ? ld_dev(&a.p_at[p0 + tid]) : 0.0;
  const uint32_t n = ld_dev(&a.lcnt[row]);
  const uint64_t k0 = ld_dev(&lkey[tid]);
  const double Atot = a.plan[row].a_above;
  const double ATtot = need_wt ? block_sum_f64(sh, vat) : Atot;
  if (tid == 0) st_dev(&a.lcnt[row], 0u);
  if (n > kCapW) {  // the window is too crowded for LDS: the row is left to nuc_alone
    if (tid == 0) a.plan[row].state = 3u;
    return;
  }
  const double tcut = (double)a.top_p * z0;
  if (n <= 64) {  // wave 0 alone, the window in its lanes
    if (tid < 64) {
      uint64_t key = (uint32_t)tid < n ? k0 : 0ull;
      uint32_t bits = (uint32_t)tid < n ? key_bits((uint32_t)(key >> 32)) : 0u;
      wave_sort(key, bits, n, F.key, s_bits);
      const bool live = (uint32_t)tid < n;
      const double w1 = live ? S1.w(__uint_as_float(bits)) : 0.0;
      const uint32_t jc = wave_pick(Atot + wave_incl_f64(w1) >= tcut, w1 > 0.0, n);
      const uint64_t kf = max(lane_key(key, jc), c.kmp);
      const uint32_t nk = (uint32_t)__builtin_popcountll(__ballot(live && key >= kf));
      const NucSet S2 = value_set(c.m, c.thr, kf, (double)a.T, e2);
      const double w2 = (uint32_t)tid < nk ? S2.w(__uint_as_float(bits)) : 0.0;
      const double wt = ATtot + wave_sum_f64(w2);
      if (tid == 0) {
        a.out_kfl[row] = kf;
        a.out_lse_f[row] = c.m / (double)a.T + log(wt);
        a.plan[row].state = 2u;
      }
    }
    return;
  }
  {  // the keys into LDS, all loads issued first
    constexpr int Q = kCapW / NT;
    uint64_t k[Q];
#pragma unroll
    for (int q = 1; q < Q; ++q) {
      const uint32_t j = q * NT + tid;
      if (j < n) k[q] = ld_dev(&lkey[j]);
    }
    if ((uint32_t)tid < n) F.key[tid] = k0;
#pragma unroll
    for (int q = 1; q < Q; ++q) {
      const uint32_t j = q * NT + tid;
      if (j < n) F.key[j] = k[q];
    }
    __syncthreads();
  }
  sort_keys_desc(F.key, n);
  const KeyBits kb{F.key};
  // the cut, then min_p: the kept candidates of the window are its first nk
  const uint32_t jc = walk_sorted(r, kb, n, S1, Atot, tcut, false);
  const uint64_t kfin = max(F.key[jc], c.kmp);
  uint32_t nk = 0;
  for (uint32_t j = tid; j < n; j += NT) nk += F.key[j] >= kfin ? 1u : 0u;
  nk = block_sum_u32(r, nk);
  const NucSet S2 = value_set(c.m, c.thr, kfin, (double)a.T, e2);
  const double WT = ATtot + sum_sorted(r, kb, nk, S2);
  if (tid == 0) {
    a.out_kfl[row] = kfin;
    a.out_lse_f[row] = c.m / (double)a.T + log(WT);
    a.plan[row].state = 2u;
  }
}

// Pass 3 (rows whose draw falls above the cut window): the exact tempered mass
// above the draw window and its candidates; the last workgroup draws.
template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void nuc_draw_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ StageOrWindow sw;
  NucLds& L = sw.L;
  Stage& st = sw.st;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  {  // both words loaded at once: most rows need nothing from this pass
    const uint32_t bad = a.st_bad[row], state = a.plan[row].state;
    if (bad || state != 1u) return;
  }
  const NucPlan p = a.plan[row];
  if (tid == 0) st.n = 0u;
  init_e2(e2);
  const NucCommon c = nuc_common(a, row, seg);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  const NucSet S1 = value_set(c.m, c.thr, 0ull, 1.0, e2, c.span1);
  const NucSet S2 = value_set(c.m, c.thr, p.kfin, (double)a.T, e2);
  uint64_t* lkey = a.lkey + row * kCapW;
  uint32_t* lbits = a.lbits + row * kCapW;
  double A2 = 0.0;
  for_each_cand<DT, VEC>(a, row, seg, p.listed != 0u, xr, c.e_begin, c.e_end, [&](uint32_t bits, int64_t i) {
    const float z = __uint_as_float(bits);
    const uint64_t K = comp_key(bits, (uint32_t)i);
    // kept candidates above the cut window
    const bool kept = z > -__builtin_inff() && (double)z >= c.thr && S1.bin<kNB>(z) < p.b_lo && K >= p.kfin;
    const uint32_t bt = kept ? S2.bin<kNB>(z) : (uint32_t)kNB;
    if (bt < p.c_lo) A2 += S2.w(z);  // (few elements: a branch)
    if (bt >= p.c_lo && bt <= p.c_hi) stage_window(st, i, c.e_begin);
  });
  flush_window<DT>(st, xr, c.e_begin, &a.lcnt[row], lkey, lbits);
  A2 = nuc_sum(r, A2, 0);
  if (tid == 0) st_dev(&a.p_a2[row * a.S + seg], A2);
  if (!last_of_row(sh, a.tickets + row * 3 + 2, (uint32_t)a.S)) return;
  const double A2tot = merge_sum(sh, a.p_a2 + row * a.S, a.S);
  const uint32_t n = ld_dev(&a.lcnt[row]);
  __syncthreads();
  if (tid == 0) st_dev(&a.lcnt[row], 0u);
  if (n > kCapW) {
    // the draw window is too crowded for LDS: the draw is left to nuc_alone
    if (tid == 0) a.plan[row].state = 4u;
    return;
  }
  take_list(L.w.key, L.w.bits, lkey, lbits, n);
  sort_window(L.w.key, L.w.bits, n);
  const uint32_t jd = walk_sorted(r, L.w.bits, n, S2, A2tot, (double)a.u[row] * p.wt, true);
  if (tid == 0) {
    a.out_token[row] = ~(uint32_t)L.w.key[jd];
    if (a.out_logp)
      a.out_logp[row] = (float)(((double)__uint_as_float(L.w.bits[jd]) - c.m) / (double)a.T - log(p.wt));
  }
}

// Rows whose window was too crowded for LDS (one workgroup per row): the
// whole row (state 3) or its draw (state 4) by the workgroup alone.
template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void nuc_alone_kernel(NucArgs a) {
  __shared__ NucRed r;
  __shared__ FbShared fb;
  __shared__ double e2[64];
  const int64_t row = blockIdx.x;
  if (row >= a.rows) return;
  const uint32_t bad = a.st_bad[row], state = a.plan[row].state;  // loaded at once
  if (bad || (state != 3u && state != 4u)) return;
  init_e2(e2);
  const NucCommon c = nuc_common(a, row, 0);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  if (state == 3u) {
    row_alone<DT, VEC>(fb, r, a, row, c, xr, e2);
    return;
  }
  const NucPlan p = a.plan[row];
  const NucSet S2 = value_set(c.m, c.thr, p.kfin, (double)a.T, e2);
  const SelOut d = wg_select<DT, VEC>(fb, r, xr, a.V, S2, (double)a.u[row], true);
  if (threadIdx.x == 0) {
    a.out_token[row] = ~(uint32_t)d.key;
    if (a.out_logp) a.out_logp[row] = (float)(((double)__uint_as_float(d.bits) - c.m) / (double)a.T - log(d.tot));
  }
}

// Typical-p over whole rows (top_k = 0) ("Chapter 21", section 21.7:
// typical_p after top_n_sigma and before top_p; ties keep the candidates' id
// order).  With p the softmax of the candidates, -log p - H = E_p[z] - z, so
// the typical order is the distance of z to the centre c = E_p[z] (then id);
// the typical set is the shortest prefix of that order whose mass reaches
// typical_p.  Then top-p in value order within it (when top_p < 1), min-p
// against its maximum, and the draw in value order (top_p < 1) or typical
// order (top_p == 1).
//
// Every decision is a weighted selection (SelJob: candidate set, order,
// weights, target), run by passes over (row, segment) workgroups:
//   typ_moments: the candidates' mass, mass-weighted value and lowest value;
//                the last workgroup sets the centre and opens the typical cut;
//   sel_hist:    guide histogram in the job's order and the exact total; the
//                last workgroup places a window around the target;
//   sel_collect: the exact mass before the window and the window's
//                candidates; the last workgroup sorts them and walks to the
//                target, or leaves the row to sel_alone when they overflow LDS;
//   sel_alone:   such rows by one workgroup (guide passes over key ranges).
// The workgroup that finishes a selection turns it into the row's next job,
// or writes the token.  The three passes run once per selection: two or three
// times.

__device__ __forceinline__ NucSet job_set(const SelJob& j, const double* e2) {
  return NucSet{j.m, j.thr, j.kfloor, j.T, e2, j.order, j.c, j.span, j.kT};
}

// The first-level span of a selection in typical order at target frac over
// candidates whose largest value is zmax: candidates farther from the centre
// c than the crossing bound lie below it (once the bound passes m - c), where
// distance d means weight at most e^((c - d - m) / T) against the heaviest
// candidate's e^((zmax - m) / T); so the bound in distance is
// T ln(n / rest) + c - zmax (crossing_depth with that lead, scaled by T).
__device__ __forceinline__ double typ_span(const SelJob& j, double frac, int64_t n, double zmax) {
  const double d = j.T * crossing_depth(frac, n, 0.0) + j.c - zmax;
  return fmin(j.span_all, fmax(d, j.m - j.c));
}

template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void typ_moments_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  if (a.st_bad[row]) {
    if (seg == 0 && tid == 0) {
      a.out_token[row] = kFail;
      if (a.out_logp) a.out_logp[row] = __builtin_nanf("");
      a.jobs[row].state = 0;
    }
    return;
  }
  init_e2(e2);
  const NucCommon c = nuc_common(a, row, seg);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  double z0 = 0.0, y = 0.0, zlo = c.m;
  for_each_elem<DT, kNG, VEC>(xr, c.e_begin, c.e_end, [&](uint32_t bits, int64_t) {
    const float z = __uint_as_float(bits);
    const bool ok = z > -__builtin_inff() && (double)z >= c.thr;
    const double e = exp_le0((double)z - c.m, e2);  // taken either way (no branch)
    const double w = ok ? e : 0.0, zd = ok ? (double)z : 0.0;
    z0 += w;
    y += w * zd;
    zlo = fmin(zlo, ok ? zd : zlo);
  });
  z0 = nuc_sum(r, z0, 0);
  y = nuc_sum(r, y, 1);
  zlo = block_ext_f64<false>(r, zlo);
  const int64_t p0 = row * a.S;
  if (tid == 0) {
    st_dev(&a.p_z0[p0 + seg], z0);
    st_dev(&a.p_a[p0 + seg], y);
    st_dev(&a.p_at[p0 + seg], zlo);
  }
  if (!last_of_row(sh, a.tickets + row * 3, (uint32_t)a.S)) return;
  const double Z0 = merge_sum(sh, a.p_z0 + p0, a.S), Y = merge_sum(sh, a.p_a + p0, a.S);
  const double lo = block_ext_f64<false>(r, tid < a.S ? ld_dev(&a.p_at[p0 + tid]) : c.m);
  if (tid == 0) {
    const double cen = Y / Z0;
    SelJob& j = a.jobs[row];
    j.m = c.m;
    j.thr = c.thr;
    j.T = 1.0;
    j.c = cen;
    j.span_all = fmax(fmax(c.m - cen, cen - lo), 1e-30) * (1.0 + 1e-6);
    j.span = typ_span(j, (double)a.typical_p, a.V, c.m);
    j.tot_known = Z0;  // the typical order's weights are these: the guide pass needs no exact sums
    j.listed = 0u;
    j.frac = (double)a.typical_p;
    j.kfloor = 0ull;
    j.kT = 0ull;
    j.order = 1;
    j.strict = 0;
    j.step = 1;
    j.state = 1;
  }
}

// A finished selection (state 4) becomes the row's next job, or its token.
__device__ void typ_advance(const NucArgs& a, int64_t row, SelJob& j) {
  if (j.step == 1) {
    // the typical set: score keys >= the cut's; its maximum is the min_p reference
    j.kT = j.key;
    j.aux = j.zmax;
    if (a.top_p < 1.0f) {
      j.order = 0;  // top-p in value order within the set, untempered
      j.T = 1.0;
      j.frac = (double)a.top_p;
      j.strict = 0;
      j.step = 2;
      j.span = fmin(kSpan, crossing_depth(j.frac, a.V, j.m - j.aux));
      j.tot_known = j.cum;  // the typical set's mass
    } else {
      if (a.min_p > 0.0f) j.thr = fmax(j.thr, j.aux + log((double)a.min_p));
      j.T = (double)a.T;  // the draw in typical order
      j.frac = (double)a.u[row];
      j.strict = 1;
      j.step = 3;
      j.span = typ_span(j, j.frac, a.V, j.aux);
      j.tot_known = a.T == 1.0f && a.min_p == 0.0f ? j.cum : 0.0;  // (the same set and weights)
    }
    j.state = 1;
  } else if (j.step == 2) {
    uint64_t kfin = j.key;
    if (a.min_p > 0.0f) kfin = max(kfin, key_floor(j.aux + log((double)a.min_p)));
    j.kfloor = kfin;  // the draw in value order over the kept set
    j.T = (double)a.T;
    j.frac = (double)a.u[row];
    j.strict = 1;
    j.step = 3;
    j.span = fmin(kSpan, crossing_depth(j.frac, a.V, (j.m - j.aux) / j.T));
    j.tot_known = a.T == 1.0f && a.min_p == 0.0f ? j.cum : 0.0;  // (the same set and weights)
    j.state = 1;
  } else {
    a.out_token[row] = key_id(j.order, j.key);
    if (a.out_logp) a.out_logp[row] = (float)(((double)__uint_as_float(j.bits) - j.m) / j.T - log(j.tot));
    j.state = 0;
  }
}

// The guide pass of a selection.  The first selection (the typical cut) also
// gathers its candidates within the crossing bound per segment; when they all
// fit and its window stays short of the last bin, they hold every candidate
// of the later selections too (the typical set precedes the selected
// candidate in the typical order), and the later passes visit only them.
template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void sel_hist_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ NucLds L;
  __shared__ GatherStage gs;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows || a.jobs[row].state != 1) return;
  const SelJob jb = a.jobs[row];
  init_e2(e2);
  const NucSet S = job_set(jb, e2);
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  for (int b = tid; b < kNB; b += NT) {
    L.h.hw[b] = 0.0;
    L.h.hc[b] = 0u;
  }
  __syncthreads();
  double t = 0.0, dw = 0.0;
  uint32_t dn = 0, ng = 0;
  const bool known = jb.tot_known > 0.0, first = jb.step == 1, listed = !first && jb.listed != 0u;
  by_order(S.order, [&](auto ord) {
    if (known) {
      // the exact total is known: float32 guide weights, and none for the
      // candidates past the crossing bound (the last bin needs only their count)
      for_each_cand<DT, VEC>(a, row, seg, listed, xr, e_begin, e_end, [&](uint32_t bits, int64_t i) {
        uint64_t K;
        uint32_t b;
        const bool ok = S.look<kNB, decltype(ord)::value>(bits, (uint32_t)i, K, b);
        const bool shallow = ok && b < kNB - 1;
        if (shallow) {
          __hip_atomic_fetch_add(&L.h.hw[b], (double)S.gw(__uint_as_float(bits)), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_add(&L.h.hc[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (first) gather(gs, ng, shallow, i, e_begin, bits);
        dn += ok && b == kNB - 1 ? 1u : 0u;
      });
      return;
    }
    for_each_cand<DT, VEC>(a, row, seg, listed, xr, e_begin, e_end, [&](uint32_t bits, int64_t i) {
      uint64_t K;
      uint32_t b;
      const bool ok = S.look<kNB, decltype(ord)::value>(bits, (uint32_t)i, K, b);
      if (ok) {  // (a subset of the row: a branch)
        const double w = S.w(__uint_as_float(bits));
        if (b < kNB - 1) {
          __hip_atomic_fetch_add(&L.h.hw[b], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_add(&L.h.hc[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
          dw += w;
          ++dn;
        }
        t += w;
      }
      if (first) gather(gs, ng, ok && b < kNB - 1, i, e_begin, bits);
    });
  });
  add_deep(L.h.hw, L.h.hc, dw, dn);
  if (first) flush_gather(gs, ng, e_begin, a, row, seg);
  __syncthreads();
  double* gw = a.h0w + row * kNB;
  uint32_t* gc = a.h0c + row * kNB;
  uint32_t* htop = &a.jobs[row].htop;
  flush_hist(L.h.hw, L.h.hc, gw, gc, htop);
  if (!known) {
    t = nuc_sum(r, t, 0);
    if (tid == 0) st_dev(&a.p_z0[row * a.S + seg], t);
  }
  if (!last_of_row(sh, a.tickets + row * 3, (uint32_t)a.S)) return;
  // ---- the row's last workgroup: its global loads issued together
  const int64_t p0 = row * a.S;
  const double vt = !known && tid < a.S ? ld_dev(&a.p_z0[p0 + tid]) : 0.0;
  const int vg = first && tid < a.S ? (int)ld_dev(&a.gcnt[p0 + tid]) : 0;
  double hv[kHQ];
  uint32_t hcv[kHQ];
  load_hist(gw, gc, hv, hcv);
  const double tot = known ? jb.tot_known : block_sum_f64(sh, vt);
  const bool fit = block_max_i32(r, vg) <= kGatherCap;
  put_hist(L.h.hw, L.h.hc, hv, hcv);
  const double tg = jb.frac * tot, g = kGuard * tot;
  pick_bins<kNB>(r, L.h.hw, L.h.hc, kNB, 0.0, tg - g, tg + g);
  const bool now_listed = first ? fit && r.b_hi < (uint32_t)kNB - 1 : jb.listed != 0u;
  if (tid == 0) {
    SelJob& j = a.jobs[row];
    j.b_lo = r.cnt_top <= kCapW ? 0u : r.b_lo;  // from the front of the order when it fits
    j.b_hi = r.b_hi;
    j.tot = tot;
    j.listed = now_listed ? 1u : 0u;
    j.state = 2;
  }
  clear_hist(gw, gc, htop);
}

template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void sel_collect_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ StageOrWindow sw;
  NucLds& L = sw.L;
  Stage& st = sw.st;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows || a.jobs[row].state != 2) return;
  const SelJob jb = a.jobs[row];
  if (tid == 0) st.n = 0u;
  init_e2(e2);
  const NucSet S = job_set(jb, e2);
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  uint64_t* lkey = a.lkey + row * kCapW;
  uint32_t* lbits = a.lbits + row * kCapW;
  double A = 0.0, zb = -__builtin_inf();  // mass and largest value before the window
  by_order(S.order, [&](auto ord) {
    for_each_cand<DT, VEC>(a, row, seg, jb.listed != 0u, xr, e_begin, e_end, [&](uint32_t bits, int64_t i) {
      uint64_t K;
      uint32_t b;
      const bool ok = S.look<kNB, decltype(ord)::value>(bits, (uint32_t)i, K, b);
      const float z = __uint_as_float(bits);
      if (!ok) return;
      if (b < jb.b_lo) {  // (few elements: a branch)
        A += S.w(z);
        zb = fmax(zb, (double)z);
      } else if (b <= jb.b_hi) {
        stage_window(st, i, e_begin);
      }
    });
  });
  flush_window<DT>(st, xr, e_begin, &a.lcnt[row], lkey, lbits, &S);
  A = nuc_sum(r, A, 0);
  zb = block_ext_f64<true>(r, zb);
  const int64_t p0 = row * a.S;
  if (tid == 0) {
    st_dev(&a.p_a[p0 + seg], A);
    st_dev(&a.p_at[p0 + seg], zb);
  }
  if (!last_of_row(sh, a.tickets + row * 3, (uint32_t)a.S)) return;
  // ---- the row's last workgroup: its first global loads issued together
  const double va = tid < a.S ? ld_dev(&a.p_a[p0 + tid]) : 0.0;
  const double vb = tid < a.S ? ld_dev(&a.p_at[p0 + tid]) : -__builtin_inf();
  const uint32_t n = ld_dev(&a.lcnt[row]);
  const uint64_t k0 = ld_dev(&lkey[tid]);
  const uint32_t b0 = ld_dev(&lbits[tid]);
  const double Atot = block_sum_f64(sh, va);
  const double zbt = block_ext_f64<true>(r, vb);
  if (tid == 0) st_dev(&a.lcnt[row], 0u);
  if (n > kCapW) {
    if (tid == 0) a.jobs[row].state = 3;  // too crowded for LDS: left to sel_alone
    return;
  }
  if (n <= 64) {
    // a small window: the selection by wave 0 alone, the window in its lanes
    if (tid < 64) {
      uint64_t key = (uint32_t)tid < n ? k0 : 0ull;
      uint32_t bits = (uint32_t)tid < n ? b0 : 0u;
      wave_sort(key, bits, n, L.w.key, L.w.bits);
      const bool live = (uint32_t)tid < n;
      const double w = live ? S.w(__uint_as_float(bits)) : 0.0;
      const double cw = Atot + wave_incl_f64(w), tg = jb.frac * jb.tot;
      const uint32_t j = wave_pick(jb.strict ? (tg < cw) : (cw >= tg), w > 0.0, n);
      // the largest value among the window's candidates up to the selected one
      double zl = live && (uint32_t)tid <= j ? (double)__uint_as_float(bits) : -__builtin_inf();
      for (int d = 1; d < 64; d <<= 1) zl = fmax(zl, __shfl_xor(zl, d));
      if ((uint32_t)tid == j) {
        SelJob& o = a.jobs[row];
        o.key = key;
        o.bits = bits;
        o.zmax = fmax(zbt, zl);
        o.cum = cw;
        o.state = 4;
        typ_advance(a, row, o);
      }
    }
    return;
  }
  take_list_pf(L.w.key, L.w.bits, lkey, lbits, n, k0, b0);
  sort_window(L.w.key, L.w.bits, n);
  double cum = 0.0;
  const uint32_t j = walk_sorted(r, L.w.bits, n, S, Atot, jb.frac * jb.tot, jb.strict != 0, &cum);
  double zl = -__builtin_inf();  // the window's candidates up to the selected one
  for (uint32_t q = tid; q <= j && q < n; q += NT) zl = fmax(zl, (double)__uint_as_float(L.w.bits[q]));
  zl = block_ext_f64<true>(r, zl);
  if (tid == 0) {
    SelJob& o = a.jobs[row];
    o.key = L.w.key[j];
    o.bits = L.w.bits[j];
    o.zmax = fmax(zbt, zl);
    o.cum = cum;
    o.state = 4;
    typ_advance(a, row, o);
  }
}

template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void sel_alone_kernel(NucArgs a) {
  __shared__ NucRed r;
  __shared__ FbShared fb;
  __shared__ double e2[64];
  const int64_t row = blockIdx.x;
  if (row >= a.rows || a.jobs[row].state != 3) return;
  const SelJob jb = a.jobs[row];
  init_e2(e2);
  const NucSet S = job_set(jb, e2);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  const SelOut d = wg_select<DT, VEC>(fb, r, xr, a.V, S, jb.frac, jb.strict != 0);
  double zl = -__builtin_inf();
  for_each_elem<DT, kNG, VEC>(xr, 0, a.V, [&](uint32_t bits, int64_t i) {
    const uint64_t K = S.key(bits, (uint32_t)i);
    if (K >= d.key && S.in(bits, (uint32_t)i, K)) zl = fmax(zl, (double)__uint_as_float(bits));
  });
  zl = block_ext_f64<true>(r, zl);
  if (threadIdx.x == 0) {
    SelJob& o = a.jobs[row];
    o.key = d.key;
    o.bits = d.bits;
    o.tot = d.tot;
    o.zmax = zl;
    o.cum = d.cum;
    o.state = 4;
    typ_advance(a, row, o);
  }
}

template <typename DT, bool VEC>
static void go_typical(const NucArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.S)), one((unsigned)a.rows);
  hipLaunchKernelGGL((typ_moments_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
  const int nsel = a.top_p < 1.0f ? 3 : 2;
  for (int q = 0; q < nsel; ++q) {
    hipLaunchKernelGGL((sel_hist_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
    hipLaunchKernelGGL((sel_collect_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
    hipLaunchKernelGGL((sel_alone_kernel<DT, VEC>), one, dim3(NT), 0, s, a);
  }
}

hipError_t launch_row_typical(int dtype, const NucArgs& a, hipStream_t s) {
  if (dtype == 0)
    a.vec ? go_typical<float, true>(a, s) : go_typical<float, false>(a, s);
  else
    a.vec ? go_typical<uint16_t, true>(a, s) : go_typical<uint16_t, false>(a, s);
  return hipGetLastError();
}

// Floor mode with min_p only: the kept set is z >= max + log(min_p); its
// log sum of exp(z/T) in float64 (fixed order), per (row, segment).
template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void kept_lse_kernel(NucArgs a) {
  __shared__ SelShared sh;
  __shared__ NucRed r;
  __shared__ double e2[64];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  if (a.st_bad[row]) {
    if (seg == 0 && tid == 0) {
      a.out_kfl[row] = 0ull;
      a.out_lse_f[row] = __builtin_nan("");
    }
    return;
  }
  init_e2(e2);
  const DT* __restrict__ xr = nuc_row<DT>(a, row);
  const double m = a.st_max[row], T = a.T, iT = 1.0 / T;
  const double thr = m + log((double)a.min_p);
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);
  double w = 0.0;
  for_each_elem<DT, kNG, VEC>(xr, e_begin, e_end, [&](uint32_t bits, int64_t) {
    const float z = __uint_as_float(bits);
    const double e = exp_le0(((double)z - m) * iT, e2);  // taken either way (no branch)
    w += (double)z >= thr ? e : 0.0;
  });
  w = nuc_sum(r, w, 0);
  if (a.S > 1) {
    if (tid == 0) st_dev(&a.p_z0[row * a.S + seg], w);
    if (!last_of_row(sh, a.tickets + row, (uint32_t)a.S)) return;
    w = merge_sum(sh, a.p_z0 + row * a.S, a.S);
  }
  if (tid == 0) {
    a.out_kfl[row] = key_floor(thr);
    a.out_lse_f[row] = m / T + log(w);
  }
}

hipError_t launch_kept_lse(int dtype, const NucArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.S));
  if (dtype == 0) {
    if (a.vec)
      hipLaunchKernelGGL((kept_lse_kernel<float, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((kept_lse_kernel<float, false>), grid, dim3(NT), 0, s, a);
  } else {
    if (a.vec)
      hipLaunchKernelGGL((kept_lse_kernel<uint16_t, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((kept_lse_kernel<uint16_t, false>), grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

template <typename DT, bool VEC>
static void go_nucleus(const NucArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.S));
  hipLaunchKernelGGL((nuc_hist_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
  if (a.out_kfl)
    hipLaunchKernelGGL((nuc_collect_floor_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((nuc_collect_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
  hipLaunchKernelGGL((nuc_draw_kernel<DT, VEC>), grid, dim3(NT), 0, s, a);
  hipLaunchKernelGGL((nuc_alone_kernel<DT, VEC>), dim3((unsigned)a.rows), dim3(NT), 0, s, a);
}

hipError_t launch_row_nucleus(int dtype, const NucArgs& a, hipStream_t s) {
  if (dtype == 0)
    a.vec ? go_nucleus<float, true>(a, s) : go_nucleus<float, false>(a, s);
  else
    a.vec ? go_nucleus<uint16_t, true>(a, s) : go_nucleus<uint16_t, false>(a, s);
  return hipGetLastError();
}

}  // namespace vsel
