// Stand-ins for the library's kernel launchers, linked with the host half of
// the C ABI (csrc/api.cpp) in place of the HIP kernels, for a host build under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing runs on a device:
// each stand-in checks on the host the launch the real launcher would make --
// the segment plan covers the row with no empty segment and respects the
// kernel's limits, and every workspace array the kernel addresses (at the
// extents its argument block documents) lies inside the workspace the driver
// declared, apart from the launch's other arrays -- then returns success.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../vocab_row_reductions_amd/csrc/internal.hpp"

namespace stub {
uintptr_t ws_lo = 0, ws_hi = 0;  // the workspace of the call under test
long launches = 0, failures = 0;

void fail(const char* what, const char* field) {
  ++failures;
  std::fprintf(stderr, "launch check failed: %s: %s\n", what, field);
}

// The workspace arrays of the launch being checked, [begin, end) with names.
struct Span {
  uintptr_t b, e;
  const char* field;
};
std::vector<Span> spans;

// a workspace array of n elements of T at p
template <class T>
void in_ws(const char* what, const char* field, const T* p, int64_t n) {
  if (!p) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (n < 0 || a < ws_lo || a + (uintptr_t)n * sizeof(T) > ws_hi || a % alignof(T) != 0) fail(what, field);
  if (n > 0) spans.push_back(Span{a, a + (uintptr_t)n * sizeof(T), field});
}

// no two arrays of one launch overlap
void disjoint(const char* what) {
  for (size_t i = 0; i < spans.size(); ++i)
    for (size_t j = i + 1; j < spans.size(); ++j)
      if (spans[i].b < spans[j].e && spans[j].b < spans[i].e) {
        std::fprintf(stderr, "overlap of %s and %s\n", spans[i].field, spans[j].field);
        fail(what, "arrays overlap");
      }
  spans.clear();
}

void plan(const char* what, int64_t V, int64_t seg_len, int32_t S, int64_t granule) {
  if (S < 1 || S > vsel::kMaxSegments || seg_len < 1 || seg_len % granule != 0 || seg_len * S < V ||
      seg_len * (S - 1) >= V)
    fail(what, "segment plan");
}
}  // namespace stub

namespace vsel {
using namespace stub;

static hipError_t check_scan(const ScanArgs& a) {
  ++launches;
  const int64_t rows = a.rows1 + a.rows2, n = rows * a.S;
  plan("scan", a.V, a.seg_len, a.S, 8);
  in_ws("scan", "tickets", a.tickets, rows);
  in_ws("scan", "p_key", a.p_key, n);
  in_ws("scan", "p_m", a.p_m, n);
  in_ws("scan", "p_s", a.p_s, n);
  for (const uint32_t* p : {a.st_amax, a.st_bad}) in_ws("scan", "row stats", p, rows);
  in_ws("scan", "st_max", a.st_max, rows);
  in_ws("scan", "st_lse", a.st_lse, rows);
  in_ws("scan", "m_n", a.m_n, n);
  in_ws("scan", "m_mean", a.m_mean, n);
  in_ws("scan", "m_m2", a.m_m2, n);
  in_ws("scan", "sigma", a.sigma, rows);
  if (a.sigma && (a.n_excl > 0 || !a.m_n || !a.m_mean || !a.m_m2)) fail("scan", "row moments");
  disjoint("scan");
  return hipSuccess;
}

hipError_t launch_scan(int, bool, const ScanArgs& a, hipStream_t) { return check_scan(a); }

static hipError_t check_topk(const TopkArgs& a, int cap) {
  ++launches;
  const int64_t n = a.rows * a.S, nr = a.S > 1 ? n * a.k : 0;
  plan("topk", a.V, a.seg_len, a.S, 8);
  if (a.k < 1 || a.k > a.V || (int64_t)a.S * a.k > cap) fail("topk", "k and the merge buffer");
  in_ws("topk", "tickets", a.tickets, a.rows);
  in_ws("topk", "rec_key", a.rec_key, nr);
  in_ws("topk", "rec_bits", a.rec_bits, nr);
  in_ws("topk", "rec_cnt", a.rec_cnt, n);
  in_ws("topk", "p_m", a.p_m, n);
  in_ws("topk", "p_s", a.p_s, n);
  in_ws("topk", "m_n", a.m_n, n);
  in_ws("topk", "m_mean", a.m_mean, n);
  in_ws("topk", "m_m2", a.m_m2, n);
  disjoint("topk");
  return hipSuccess;
}

hipError_t launch_topk(int, bool, int cap, const TopkArgs& a, hipStream_t) {
  if (a.m_n) fail("topk", "row moments outside the per-wave kernel");
  return check_topk(a, cap);
}
hipError_t launch_topk_wave(int, bool, const TopkArgs& a, hipStream_t) {
  if (a.k > kWaveTopkMax || !a.vec) fail("topk_wave", "k or alignment");
  return check_topk(a, kCapSmall);
}
int topk_wave_blocks_per_cu(int, bool) { return 4; }
int scan_blocks_per_cu(int, bool) { return 4; }
int topk_blocks_per_cu(int, bool, int cap) { return cap == kCapSmall ? 4 : 2; }

static void check_spec(const char* what, const SpecArgs& a) {
  ++launches;
  const int64_t B = a.B, G = a.gamma, nrows = B * (2 * G + 1);
  plan(what, a.V, a.seg_len, a.S, 8);
  plan(what, a.V, a.dseg, a.dS, kChunk);
  if (a.dseg > (int64_t)kChunk * kChunksPerSeg || a.nchunk != (a.V + kChunk - 1) / kChunk) fail(what, "draw plan");
  in_ws(what, "tk_pos", a.tk_pos, B * G);
  in_ws(what, "tk_seq", a.tk_seq, B);
  in_ws(what, "tk_draw", a.tk_draw, B);
  in_ws(what, "p_summin", a.p_summin, B * G * a.S);
  in_ws(what, "acc", a.acc, B * G);
  in_ws(what, "draw_L", a.draw_L, B);
  in_ws(what, "p_lse", a.p_lse, B * 2 * a.dS);
  in_ws(what, "p_w", a.p_w, B * a.dS);
  in_ws(what, "p_c", a.p_c, B * a.nchunk);
  in_ws(what, "p_cb", a.p_cb, B * a.nchunk);
  in_ws(what, "p_cf", a.p_cf, B * a.nchunk);
  in_ws(what, "p_low", a.p_low, B * G * a.S);
  in_ws(what, "p_wt", a.p_wt, B * G * a.S);
  in_ws(what, "st_amax", a.st_amax, nrows);
  in_ws(what, "st_max", a.st_max, nrows);
  in_ws(what, "st_lse", a.st_lse, nrows);
  in_ws(what, "st_bad", a.st_bad, nrows);
  in_ws(what, "kfl", a.kfl, nrows);
  disjoint(what);
}

hipError_t launch_spec(const SpecArgs& a, hipStream_t) {
  check_spec("spec", a);
  return hipSuccess;
}
hipError_t launch_spec_match(const SpecArgs& a, hipStream_t) {
  check_spec("spec_match", a);
  return hipSuccess;
}

hipError_t launch_draw_rows(int, const DrawArgs& a, hipStream_t) {
  ++launches;
  plan("draw", a.V, a.seg_len, a.S, kChunk);
  if (a.seg_len > (int64_t)kChunk * kChunksPerSeg || a.nchunk != (a.V + kChunk - 1) / kChunk)
    fail("draw", "draw plan");
  in_ws("draw", "tickets", a.tickets, a.rows);
  in_ws("draw", "p_w", a.p_w, a.rows * a.S);
  in_ws("draw", "p_c", a.p_c, a.rows * a.nchunk);
  in_ws("draw", "st_max", a.st_max, a.rows);
  in_ws("draw", "st_bad", a.st_bad, a.rows);
  in_ws("draw", "sigma", a.sigma, a.rows);
  disjoint("draw");
  return hipSuccess;
}

hipError_t launch_moments(int, const MomArgs& a, hipStream_t) {
  ++launches;
  plan("moments", a.V, a.seg_len, a.S, 8);
  in_ws("moments", "tickets", a.tickets, a.rows);
  in_ws("moments", "p_n", a.p_n, a.rows * a.S);
  in_ws("moments", "p_mean", a.p_mean, a.rows * a.S);
  in_ws("moments", "p_m2", a.p_m2, a.rows * a.S);
  in_ws("moments", "sigma", a.sigma, a.rows);
  disjoint("moments");
  return hipSuccess;
}

static void check_nuc(const char* what, const NucArgs& a, bool full) {
  ++launches;
  plan(what, a.V, a.seg_len, a.S, 8);
  const int64_t R = a.rows, n = R * a.S;
  in_ws(what, "tickets", a.tickets, full ? 3 * R : R);
  in_ws(what, "p_z0", a.p_z0, n);
  in_ws(what, "st_max", a.st_max, R);
  in_ws(what, "st_bad", a.st_bad, R);
  in_ws(what, "out_kfl", a.out_kfl, R);
  in_ws(what, "out_lse_f", a.out_lse_f, R);
  if (a.x2 && (a.rows1 < 1 || a.rows1 >= R)) fail(what, "second batch");
  if (!full) return disjoint(what);
  in_ws(what, "h0w", a.h0w, R * kNucBins);
  in_ws(what, "h0c", a.h0c, R * kNucBins);
  in_ws(what, "hTw", a.hTw, R * kNucBins);
  in_ws(what, "hTc", a.hTc, R * kNucBins);
  in_ws(what, "lkey", a.lkey, R * kNucCap);
  in_ws(what, "lbits", a.lbits, R * kNucCap);
  in_ws(what, "lcnt", a.lcnt, R);
  in_ws(what, "gcnt", a.gcnt, n);
  in_ws(what, "gbits", a.gbits, n * kGatherCap);
  in_ws(what, "gidx", a.gidx, n * kGatherCap);
  in_ws(what, "p_a", a.p_a, n);
  in_ws(what, "p_at", a.p_at, n);
  in_ws(what, "p_a2", a.p_a2, n);
  in_ws(what, "plan", a.plan, R);
  in_ws(what, "jobs", a.jobs, R);
  in_ws(what, "sigma", a.sigma, R);
  disjoint(what);
}

hipError_t launch_row_nucleus(int, const NucArgs& a, hipStream_t) {
  check_nuc("nucleus", a, true);
  return hipSuccess;
}
hipError_t launch_kept_lse(int, const NucArgs& a, hipStream_t) {
  check_nuc("kept_lse", a, false);
  return hipSuccess;
}
hipError_t launch_row_typical(int, const NucArgs& a, hipStream_t) {
  check_nuc("typical", a, true);
  if (!a.jobs) fail("typical", "jobs");
  return hipSuccess;
}

}  // namespace vsel
