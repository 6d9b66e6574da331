// api.cpp -- the C ABI of include/vsel.h: argument checks, workspace
// layout, segment planning and kernel dispatch.  Host code only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/vsel.h"
#include "internal.hpp"

using namespace vsel;

namespace {

constexpr int64_t kMinSegment = 2048;      // elements per workgroup, at least
// A top-k segment pays a threshold start, an epilogue and its share of the
// row's merge, so shorter ones lose: on 64 x 202,048 and 3 or 49 x 248,320
// f32 rows the best plans had 8 to 11 segments (24-32 K elements), and 13
// to 16 segments ran 10-15% slower.  The moments pass (float64 pairwise
// merges of count, mean and M2) shows the same: 8 segments of a 202,048 row
// beat 16.
constexpr int64_t kMinMergeSegment = 24576;
constexpr int64_t kSegOverhead = 4096;     // fixed cost of a segment, in elements streamed
constexpr int64_t kMergePerRecord = 32;    // a record merged by a row's last workgroup, in elements streamed
constexpr int64_t kMaxSplitWork = 8192;    // rows x segments never exceeds max(rows, this)
constexpr size_t kTicketFloor = 65536;     // counters live in the first 64 KiB (or more)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int32_t S;
  int64_t seg_len;
};

// Upper bound on segments per row.  It depends on the shape only, so the
// workspace can be sized without the device: no segment shorter than
// kMinSegment, a row's k-record sets must fit one workgroup's merge buffer,
// and the split never multiplies the work items past kMaxSplitWork.
int64_t seg_bound(int64_t rows, int64_t V, int64_t k, int cap, int64_t min_seg = kMinSegment) {
  int64_t b = std::min<int64_t>(kMaxSegments, std::max<int64_t>(1, cdiv(V, min_seg)));
  if (k > 0) b = std::min<int64_t>(b, std::max<int64_t>(1, cap / k));
  return std::min<int64_t>(b, std::max<int64_t>(1, cdiv(kMaxSplitWork, rows)));
}

// Segments per row for a grid that runs `resident` workgroups at once.
// About kSatPerCu streaming workgroups per CU already saturate HBM; beyond
// that, splitting rows only adds merge work.  So a round of n workgroups
// costs (segment length + a fixed per-segment cost) x max(1, n / sat): a
// short round is bound by the workgroups' own speed, a full one by HBM.
// With k > 0 a row of S > 1 segments also pays the merge of S x k records.
// A kernel that streams `streams` rows per workgroup (target and draft)
// saturates HBM with proportionally fewer workgroups.
// Segment lengths are multiples of `granule` elements (a multiple of 8).
constexpr int64_t kSatPerCu = 4;
int device_cus();
Plan plan_segments(int64_t rows, int64_t V, int64_t k, int64_t resident, int cap, int64_t granule = 8,
                   int streams = 1, int64_t min_seg = kMinSegment) {
  const int64_t sb = seg_bound(rows, V, k, cap, min_seg);
  const int64_t sat = kSatPerCu * device_cus() / streams;
  Plan best{1, cdiv(V, granule) * granule};
  double best_cost = 1e300;
  for (int64_t S = 1; S <= sb; ++S) {
    const int64_t seg = cdiv(cdiv(V, S), granule) * granule;
    const int64_t Sx = cdiv(V, seg);
    if (Sx != S) continue;
    const int64_t n = rows * Sx, res = std::max<int64_t>(1, resident);
    double cost = 0.0;
    for (int64_t left = n; left > 0; left -= res) {
      const int64_t in_round = std::min(left, res);
      cost += (double)(seg + kSegOverhead) * std::max(1.0, (double)in_round / (double)sat);
    }
    // (8 segments of a 248,320-element verify row beat 16 by 5-13%)
    if (Sx > 1) cost += (double)(Sx * k * kMergePerRecord);
    if (cost < best_cost) {
      best_cost = cost;
      best = Plan{(int32_t)Sx, seg};
    }
  }
  return best;
}

int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int64_t resident_scan(int dtype, bool lse) {
  const int b = scan_blocks_per_cu(dtype, lse);
  return (int64_t)(b > 0 ? b : 4) * device_cus();
}
int64_t resident_topk(int dtype, bool lse, int cap) {
  const int b = topk_blocks_per_cu(dtype, lse, cap);
  return (int64_t)(b > 0 ? b : 2) * device_cus();
}

Plan plan_scan(int dtype, bool lse, int64_t rows, int64_t V, int streams = 1, int64_t min_seg = kMinSegment) {
  return plan_segments(rows, V, 0, resident_scan(dtype, lse), kCapLarge, 8, streams, min_seg);
}
Plan plan_scan_bound(int64_t rows, int64_t V) {
  const int64_t sb = seg_bound(rows, V, 0, kCapLarge);
  return Plan{(int32_t)sb, cdiv(cdiv(V, sb), 8) * 8};
}

// Draws: segments a multiple of kChunk elements, at most kChunksPerSeg
// chunks each, at most kMaxSegments per row.
constexpr int64_t kMaxDrawVocab = (int64_t)kMaxSegments * kChunk * kChunksPerSeg;
Plan plan_draw(int64_t rows, int64_t V, int64_t resident) {
  const Plan p = plan_segments(rows, V, 0, resident, kCapLarge);
  int64_t seg = cdiv(p.seg_len, kChunk) * kChunk;
  seg = std::min<int64_t>(seg, (int64_t)kChunk * kChunksPerSeg);
  seg = std::max<int64_t>(seg, cdiv(cdiv(V, kMaxSegments), kChunk) * kChunk);
  return Plan{(int32_t)cdiv(V, seg), seg};
}

// The draws of modified rejection sampling share pass 2's launch:
// about two draw workgroups per CU in all (16 segments per row for 32
// sequences), so that their float64 work spreads over the CUs beside pass 2's
// stream.  (The 32 x 8 batch: 12, 16, 24 and 32 segments per row took 158.5,
// 157.0, 171.4 and 175.8 us per call.)
Plan plan_draw_fused(int64_t B, int64_t V) {
  const int64_t want = std::min<int64_t>(kMaxSegments, std::max<int64_t>(1, cdiv(2 * device_cus(), B)));
  int64_t seg = cdiv(cdiv(V, want), kChunk) * kChunk;
  seg = std::min<int64_t>(seg, (int64_t)kChunk * kChunksPerSeg);
  seg = std::max<int64_t>(seg, cdiv(cdiv(V, kMaxSegments), kChunk) * kChunk);
  return Plan{(int32_t)cdiv(V, seg), seg};
}

// The whole-row passes (nucleus and typical-p): two workgroups per CU (LDS
// bound), each bound by its own float64 work rather than by HBM.  A CU's time
// is then its workgroups' segments plus a fixed cost per workgroup (the
// histogram flush and the row's tail, about kNucSegCost elements' worth), and
// a CU left with a single workgroup runs it at about 0.6 of the CU's rate.  S
// minimises the busiest CU's time.  (Measured on 288 speculative rows: 3
// segments 537 us per filtered call, 7 segments 558 us; 256 rows: 2 segments
// 583 us, 1 segment 633 us.)
constexpr int64_t kNucSegCost = 24576;
Plan plan_nucleus(int64_t rows, int64_t V) {
  const int64_t sb = seg_bound(rows, V, 0, kCapLarge);  // (the workspace's bound)
  const int64_t cus = device_cus();
  Plan best{1, cdiv(V, 8) * 8};
  double best_cost = 1e300;
  for (int64_t S = 1; S <= sb; ++S) {
    const int64_t seg = cdiv(cdiv(V, S), 8) * 8;
    const int64_t Sx = cdiv(V, seg);
    if (Sx != S) continue;
    const int64_t per_cu = cdiv(rows * Sx, cus);
    const double cost = (double)per_cu * (double)(seg + kNucSegCost) / (per_cu >= 2 ? 1.0 : 0.6);
    if (cost < best_cost) {
      best_cost = cost;
      best = Plan{(int32_t)Sx, seg};
    }
  }
  return best;
}

// Top-k: the small candidate buffer whenever it can hold the merge, which
// keeps four workgroups per CU.
struct TopkPlan {
  Plan p;
  int cap;
};
// Top-k segments are whole tiles (kTopkTile elements of 16 bytes per lane
// x 8 groups), so only a row's last segment ends in a partial tile.
// The per-wave variant takes k <= kWaveTopkMax on 16-byte-aligned rows.
// big_scratch: the chain's typical-p on more than kWaveTopkMax candidates,
// whose scratch needs the large buffer's free half.
TopkPlan plan_topk(int dtype, bool lse, int64_t rows, int64_t V, int64_t k, bool wave, bool big_scratch = false) {
  const int64_t tile = (int64_t)kTopkGroups * 256 * (dtype == VSEL_F32 ? 4 : 8);
  const int cap = (wave || (2 * k <= kCapSmall && !big_scratch)) ? kCapSmall : kCapLarge;
  int64_t resident = 0;
  if (wave) {
    const int b = topk_wave_blocks_per_cu(dtype, lse);
    resident = (int64_t)(b > 0 ? b : 2) * device_cus();
  } else {
    resident = resident_topk(dtype, lse, cap);
  }
  return TopkPlan{plan_segments(rows, V, k, resident, cap, tile, 1, kMinMergeSegment), cap};
}
Plan plan_topk_bound(int64_t rows, int64_t V, int64_t k) {
  const int64_t sb = seg_bound(rows, V, k, kCapLarge);
  return Plan{(int32_t)sb, 0};
}

// Sequential bump allocator over the workspace; the first region holds every
// counter the call uses (zero between calls).
struct Layout {
  size_t off = 0;
  size_t tick_bytes = 0;
  void reserve_tickets(size_t n) {
    tick_bytes = align_up(std::max(kTicketFloor, n * sizeof(uint32_t)));
    off = tick_bytes;
  }
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool elem_ok(int dtype) { return dtype == VSEL_F32 || dtype == VSEL_BF16; }
size_t elem_size(int dtype) { return dtype == VSEL_F32 ? 4 : 2; }
bool rows_ok(int64_t rows, int64_t V, int64_t ld) {
  return rows >= 1 && V >= 1 && V < (int64_t(1) << 31) && ld >= V && rows <= (int64_t(1) << 24);
}
bool aligned16(const void* p, int64_t ld, size_t es) {
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((ld * (int64_t)es) % 16 == 0);
}
bool aligned_elem(const void* p, size_t es) { return reinterpret_cast<uintptr_t>(p) % es == 0; }

// ---- layouts (the same functions size the workspace and place the buffers)
struct ScanWs {
  size_t tickets, p_key, p_m, p_s;
};
ScanWs scan_layout(Layout& L, int64_t rows, const Plan& p, bool own_tickets = true) {
  ScanWs w{};
  if (own_tickets) L.reserve_tickets((size_t)rows);
  w.tickets = 0;
  const size_t n = (size_t)(rows * p.S);
  w.p_key = L.take(n * 8);
  w.p_m = L.take(n * 4);
  w.p_s = L.take(n * 8);
  return w;
}

struct TopkWs {
  size_t tickets, rec_key, rec_bits, rec_cnt, p_m, p_s;
};
TopkWs topk_layout(Layout& L, int64_t rows, int64_t k, const Plan& p) {
  TopkWs w{};
  L.reserve_tickets((size_t)rows);
  const size_t n = (size_t)(rows * p.S);
  const size_t nr = p.S > 1 ? n * (size_t)k : 0;
  w.rec_key = L.take(nr * 8);
  w.rec_bits = L.take(nr * 4);
  w.rec_cnt = L.take(n * 4);
  w.p_m = L.take(n * 4);
  w.p_s = L.take(n * 8);
  return w;
}

struct StatsWs {
  size_t amax, mx, lse, bad;
};
StatsWs stats_layout(Layout& L, int64_t nrows) {
  StatsWs w{};
  w.amax = L.take((size_t)nrows * 4);
  w.mx = L.take((size_t)nrows * 4);
  w.lse = L.take((size_t)nrows * 8);
  w.bad = L.take((size_t)nrows * 4);
  return w;
}

// Sampling over the whole row (top_k == 0): row scan, then the draw.
struct RowDrawWs {
  ScanWs scan;
  StatsWs st;
  size_t dtickets, p_w, p_c;
};
RowDrawWs rowdraw_layout(Layout& L, int64_t rows, int64_t V, const Plan& ps) {
  RowDrawWs w{};
  L.reserve_tickets((size_t)(2 * rows));
  w.scan = scan_layout(L, rows, ps, false);
  w.scan.tickets = 0;
  w.dtickets = (size_t)rows * 4;
  w.st = stats_layout(L, rows);
  w.p_w = L.take((size_t)(rows * kMaxSegments) * 8);
  w.p_c = L.take((size_t)(rows * cdiv(V, kChunk)) * 8);
  return w;
}

struct SpecWs {
  ScanWs scan;
  StatsWs st;
  size_t tk_pos, tk_seq, tk_draw;
  size_t p_summin, acc, draw_L, p_lse, p_w, p_c, p_cb, p_cf;
  size_t p_low, p_wt;  // sampler-match
};
SpecWs spec_layout(Layout& L, int64_t B, int64_t G, int64_t V, const Plan& ps, const Plan& pp) {
  SpecWs w{};
  const int64_t nrows = B * (2 * G + 1);
  const size_t nt = (size_t)(nrows + B * G + B + B);
  L.reserve_tickets(nt);
  w.scan.tickets = 0;
  w.tk_pos = (size_t)nrows * 4;
  w.tk_seq = w.tk_pos + (size_t)(B * G) * 4;
  w.tk_draw = w.tk_seq + (size_t)B * 4;
  w.scan = scan_layout(L, nrows, ps, false);
  w.scan.tickets = 0;
  w.st = stats_layout(L, nrows);
  w.p_summin = L.take((size_t)(B * G * pp.S) * 8);
  w.acc = L.take((size_t)(B * G) * 4);
  w.draw_L = L.take((size_t)B * 4);
  w.p_lse = L.take((size_t)(2 * B * kMaxSegments) * 8);  // per draw segment
  w.p_w = L.take((size_t)(B * kMaxSegments) * 8);
  w.p_c = L.take((size_t)(B * cdiv(V, kChunk)) * 8);
  w.p_cb = L.take((size_t)(B * cdiv(V, kChunk)) * 8);
  w.p_cf = L.take((size_t)(B * cdiv(V, kChunk)) * 4);
  w.p_low = L.take((size_t)(B * G * pp.S) * 8);
  w.p_wt = L.take((size_t)(B * G * pp.S) * 8);
  return w;
}

// Workspace of the sampler for this shape (0: invalid shape).
size_t sample_ws_bytes(int64_t rows, int64_t vocab, int64_t k) {
  if (!rows_ok(rows, vocab, vocab) || k < 0 || k > VSEL_K_MAX) return 0;
  Layout a;
  scan_layout(a, rows, plan_scan_bound(rows, vocab));
  size_t need = a.off;
  if (k == 0) {
    Layout b;
    if (vocab > kMaxDrawVocab) return 0;
    rowdraw_layout(b, rows, vocab, plan_scan_bound(rows, vocab));
    need = std::max(need, b.off);
  } else if (k > 1) {
    const int64_t kk = std::min<int64_t>(k, vocab);
    Layout b;
    topk_layout(b, rows, kk, plan_topk_bound(rows, vocab, kk));
    need = std::max(need, b.off);
  }
  return need;
}

// Row moments for the chain's top-n-sigma filter, placed after the
// sampler's own workspace.
struct MomWs {
  size_t tickets, sigma, p_n, p_mean, p_m2;
};
// The whole-row nucleus passes (top_k = 0, top_p < 1).
struct NucWs {
  size_t tickets, h0w, h0c, hTw, hTc, lkey, lbits, lcnt, gcnt, gbits, gidx, p_z0, p_a, p_at, p_a2, plan, jobs;
};
NucWs nucleus_layout(Layout& L, int64_t rows, const Plan& p) {
  NucWs w{};
  const size_t R = (size_t)rows, n = (size_t)(rows * p.S);
  w.tickets = L.take(R * 3 * 4);
  w.h0w = L.take(R * kNucBins * 8);
  w.h0c = L.take(R * kNucBins * 4);
  w.hTw = L.take(R * kNucBins * 8);
  w.hTc = L.take(R * kNucBins * 4);
  w.lkey = L.take(R * kNucCap * 8);
  w.lbits = L.take(R * kNucCap * 4);
  w.lcnt = L.take(R * 4);
  w.gcnt = L.take(n * 4);
  w.gbits = L.take(n * kGatherCap * 4);
  w.gidx = L.take(n * kGatherCap * 4);
  w.p_z0 = L.take(n * 8);
  w.p_a = L.take(n * 8);
  w.p_at = L.take(n * 8);
  w.p_a2 = L.take(n * 8);
  w.plan = L.take(R * sizeof(NucPlan));
  w.jobs = L.take(R * sizeof(SelJob));
  return w;
}

MomWs moments_layout(Layout& L, int64_t rows, const Plan& p) {
  MomWs w{};
  w.tickets = L.take((size_t)rows * 4);
  w.sigma = L.take((size_t)rows * 8);
  const size_t n = (size_t)(rows * p.S);
  w.p_n = L.take(n * 8);
  w.p_mean = L.take(n * 8);
  w.p_m2 = L.take(n * 8);
  return w;
}

// The chain's regions after the sampler's own workspace: the row moments,
// and for top_k = 0 the nucleus passes.
struct ChainWs {
  MomWs mom;
  NucWs nuc;
  bool has_nuc;
};
ChainWs chain_layout(Layout& L, int64_t rows, int64_t vocab, int32_t top_k) {
  ChainWs w{};
  w.mom = moments_layout(L, rows, plan_scan_bound(rows, vocab));
  w.has_nuc = top_k == 0;
  if (w.has_nuc) w.nuc = nucleus_layout(L, rows, plan_scan_bound(rows, vocab));
  return w;
}

// Filtered speculative acceptance: after the speculative workspace, per row
// the smallest kept key and the kept set's lse (target rows, then draft
// rows), then the filter pass's scratch: a top-k workspace, used by the
// target rows and then the draft rows, and a nucleus workspace (also used by
// the min-p threshold pass) for the target and draft rows together, at its
// own 256-byte aligned base.  All are disjoint where it matters, so calls
// with any filters can share one workspace: each keeps its own counters at
// zero.
struct SpecFiltWs {
  size_t kfl, lse, sub_topk, topk_bytes, sub_nuc, end;
};
SpecFiltWs spec_filter_layout(size_t spec_end, int64_t B, int64_t G, int64_t V) {
  SpecFiltWs w{};
  const int64_t nT = B * (G + 1), nrows = B * (2 * G + 1);
  Layout L;
  L.off = align_up(spec_end);
  w.kfl = L.take((size_t)nrows * 8);
  w.lse = L.take((size_t)nrows * 8);
  // The top-k passes of the two parts (target rows, draft rows) share one
  // region: its only zero-required words, the tickets, lead every top-k
  // layout, so each part's tickets lie in the other's.  The nucleus passes
  // (and the min-p threshold pass) run over both parts in one set of
  // launches, with a region of their own.
  size_t tk = 0;
  const int64_t part_rows[2] = {nT, B * G};
  for (int part = 0; part < 2; ++part) {
    const int64_t rows = part_rows[part];
    for (int64_t k = 1; k <= std::min<int64_t>(VSEL_K_MAX, V); ++k) {
      Layout b;
      topk_layout(b, rows, k, plan_topk_bound(rows, V, k));
      tk = std::max(tk, b.off);
    }
  }
  Layout nb;
  nucleus_layout(nb, nrows, plan_scan_bound(nrows, V));
  w.sub_topk = L.take(tk);
  w.topk_bytes = tk;
  w.sub_nuc = L.take(nb.off);
  w.end = L.off;
  return w;
}

bool ws_ok(void* ws, size_t have, size_t need) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) % kWsAlign == 0) && have >= need;
}

vsel_status launched(hipError_t e) { return e == hipSuccess ? VSEL_OK : VSEL_EDEVICE; }

ScanArgs scan_args(const void* x, int dtype, int64_t rows, int64_t V, int64_t ld, const Plan& p, double T) {
  ScanArgs a{};
  a.x1 = x;
  a.x2 = nullptr;
  a.ld1 = ld;
  a.ld2 = ld;
  a.rows1 = rows;
  a.rows2 = 0;
  a.V = V;
  a.seg_len = p.seg_len;
  a.S = p.S;
  a.vec1 = aligned16(x, ld, elem_size(dtype)) ? 1 : 0;
  a.vec2 = 0;
  a.T = T > 0 ? T : 1.0;
  a.lse_c = (float)(1.4426950408889634 / a.T);
  return a;
}

}  // namespace

extern "C" {

int vsel_version(void) { return (1 << 16) | 0; }

const char* vsel_status_string(int s) {
  switch (s) {
    case VSEL_OK: return "ok";
    case VSEL_EINVAL: return "invalid argument";
    case VSEL_EWORKSPACE: return "workspace too small or misaligned";
    case VSEL_EDEVICE: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t vsel_workspace_bytes(int op, int dtype, int64_t rows, int64_t vocab, int32_t k) {
  if (!elem_ok(dtype)) return 0;
  Layout L;
  switch (op) {
    case VSEL_OP_ARGMAX: {
      if (!rows_ok(rows, vocab, vocab)) return 0;
      scan_layout(L, rows, plan_scan_bound(rows, vocab));
      return L.off;
    }
    case VSEL_OP_TOPK: {
      if (!rows_ok(rows, vocab, vocab) || k < 1 || k > VSEL_K_MAX || k > vocab) return 0;
      topk_layout(L, rows, k, plan_topk_bound(rows, vocab, k));
      return L.off;
    }
    case VSEL_OP_SAMPLE:  // the chain's layout: top_k == 0 with top_p < 1 runs the whole-row nucleus
    case VSEL_OP_SAMPLE_CHAIN: {
      const size_t base = sample_ws_bytes(rows, vocab, k);
      if (base == 0) return 0;
      L.off = align_up(base);
      chain_layout(L, rows, vocab, k);
      return L.off;
    }
    case VSEL_OP_SPEC_ACCEPT:
    case VSEL_OP_SPEC_FILTERED: {
      const int64_t B = rows, G = k;
      if (B < 1 || G < 1 || G > kMaxSegments || vocab > kMaxDrawVocab || !rows_ok(B * (2 * G + 1), vocab, vocab))
        return 0;
      spec_layout(L, B, G, vocab, plan_scan_bound(B * (2 * G + 1), vocab), plan_scan_bound(B * G, vocab));
      if (op == VSEL_OP_SPEC_ACCEPT) return L.off;
      return spec_filter_layout(L.off, B, G, vocab).end;
    }
    default:
      return 0;
  }
}

vsel_status vsel_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                        uint32_t* out_idx, float* out_val, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !out_idx || !elem_ok(dtype) || !rows_ok(rows, vocab, ld) ||
      !aligned_elem(logits, elem_size(dtype)))
    return VSEL_EINVAL;
  Layout L;
  const ScanWs w = scan_layout(L, rows, plan_scan_bound(rows, vocab));
  if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
  const Plan p = plan_scan(dtype, false, rows, vocab);
  ScanArgs a = scan_args(logits, dtype, rows, vocab, ld, p, 1.0);
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.tickets = at<uint32_t>(ws, w.tickets);
  a.p_key = at<uint64_t>(ws, w.p_key);
  a.p_m = at<float>(ws, w.p_m);
  a.p_s = at<double>(ws, w.p_s);
  return launched(launch_scan(dtype, false, a, (hipStream_t)stream));
}

vsel_status vsel_argmax_excluding(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                                  const uint32_t* excluded, int32_t n_excluded, uint32_t* out_idx,
                                  uint32_t* out_status, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !out_idx || !out_status || !elem_ok(dtype) || !rows_ok(rows, vocab, ld) ||
      !aligned_elem(logits, elem_size(dtype)) || n_excluded < 0 || n_excluded > kMaxExcluded ||
      (n_excluded > 0 && !excluded))
    return VSEL_EINVAL;
  Layout L;
  const ScanWs w = scan_layout(L, rows, plan_scan_bound(rows, vocab));
  if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
  const Plan p = plan_scan(dtype, false, rows, vocab);
  ScanArgs a = scan_args(logits, dtype, rows, vocab, ld, p, 1.0);
  a.out_idx = out_idx;
  a.out_status = out_status;
  a.excl = excluded;
  a.n_excl = n_excluded;
  a.tickets = at<uint32_t>(ws, w.tickets);
  a.p_key = at<uint64_t>(ws, w.p_key);
  a.p_m = at<float>(ws, w.p_m);
  a.p_s = at<double>(ws, w.p_s);
  return launched(launch_scan(dtype, false, a, (hipStream_t)stream));
}

// exact_layout: place the buffers for this call's own segment plan rather
// than for the shape's bound (the plan's segment count never exceeds the
// bound, so this layout is never larger; the tickets lead either layout).
static vsel_status topk_common(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                               int32_t k, bool want_lse, TopkArgs& a, void* ws, size_t ws_bytes,
                               void* stream, bool exact_layout = false) {
  const bool vec = aligned16(logits, ld, elem_size(dtype));
  const bool wave = vec && k <= kWaveTopkMax;
  const TopkPlan tp = plan_topk(dtype, want_lse, rows, vocab, k, wave, a.mode == 1 && a.typical_p < 1.0f);
  const Plan& p = tp.p;
  Layout L;
  const TopkWs w = topk_layout(L, rows, k, exact_layout ? p : plan_topk_bound(rows, vocab, k));
  if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
  a.x = logits;
  a.ld = ld;
  a.rows = rows;
  a.V = vocab;
  a.seg_len = p.seg_len;
  a.S = p.S;
  a.k = k;
  a.vec = vec ? 1 : 0;
  a.tickets = at<uint32_t>(ws, w.tickets);
  a.rec_key = at<uint64_t>(ws, w.rec_key);
  a.rec_bits = at<uint32_t>(ws, w.rec_bits);
  a.rec_cnt = at<uint32_t>(ws, w.rec_cnt);
  a.p_m = at<float>(ws, w.p_m);
  a.p_s = at<double>(ws, w.p_s);
  if (wave) return launched(launch_topk_wave(dtype, want_lse, a, (hipStream_t)stream));
  return launched(launch_topk(dtype, want_lse, tp.cap, a, (hipStream_t)stream));
}

vsel_status vsel_topk(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k,
                      float* out_vals, uint32_t* out_ids, uint32_t* out_argmax, float* out_lse, void* ws,
                      size_t ws_bytes, void* stream) {
  return (vsel_status)vsel::topk_entry(logits, dtype, rows, vocab, ld, k, out_vals, out_ids, out_argmax, out_lse,
                                       ws, ws_bytes, stream, false);
}

// The sampler (vsel_sample) and the ordered chain (vsel_sample_chain): the
// greedy short-circuit, the whole-row draw (top_k == 0; threshold filters
// only) or the top-k kernel with the chain on its candidates.  mom: where the
// row moments go (the chain, whose caller has checked the whole workspace);
// with top_n_sigma > 0 their pass runs first.
static vsel_status sample_impl(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                               float temperature, int32_t top_k, float top_p, float top_n_sigma, float typical_p,
                               float min_p, const ChainWs* cw, const float* u, uint32_t* out_token,
                               float* out_logprob, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !u || !out_token || !elem_ok(dtype) || !rows_ok(rows, vocab, ld) ||
      !aligned_elem(logits, elem_size(dtype)))
    return VSEL_EINVAL;
  if (!(temperature >= 0.0f) || std::isinf(temperature) || top_k < 0 || top_k > VSEL_K_MAX ||
      !(top_p > 0.0f && top_p <= 1.0f))
    return VSEL_EINVAL;
  if (top_k == 0 && (typical_p < 1.0f || top_p < 1.0f) && !(cw && cw->has_nuc)) return VSEL_EINVAL;
  if (top_n_sigma > 0.0f && !cw) return VSEL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const bool greedy = temperature == 0.0f || top_k == 1;

  const double* sigma = nullptr;
  // the per-wave top-k kernel takes the row moments in its own pass
  const bool fused_moments = top_n_sigma > 0.0f && !greedy && top_k > 0 &&
                             aligned16(logits, ld, elem_size(dtype)) &&
                             std::min<int64_t>(top_k, vocab) <= kWaveTopkMax;
  // over whole rows (top_k = 0) the row scan takes them in its pass
  const bool scan_moments = top_n_sigma > 0.0f && !greedy && top_k == 0;
  if (top_n_sigma > 0.0f && !greedy && !fused_moments && !scan_moments) {
    const Plan p = plan_scan(dtype, false, rows, vocab, 1, kMinMergeSegment);
    MomArgs m{};
    m.x = logits;
    m.vec = aligned16(logits, ld, elem_size(dtype)) ? 1 : 0;
    m.ld = ld;
    m.rows = rows;
    m.V = vocab;
    m.seg_len = p.seg_len;
    m.S = p.S;
    m.tickets = at<uint32_t>(ws, cw->mom.tickets);
    m.p_n = at<double>(ws, cw->mom.p_n);
    m.p_mean = at<double>(ws, cw->mom.p_mean);
    m.p_m2 = at<double>(ws, cw->mom.p_m2);
    m.sigma = at<double>(ws, cw->mom.sigma);
    if (launch_moments(dtype, m, s) != hipSuccess) return VSEL_EDEVICE;
    sigma = m.sigma;
  }

  if (greedy) {
    // Greedy: the argmax, nothing drawn; log-probability 0.
    Layout L;
    const ScanWs w = scan_layout(L, rows, plan_scan_bound(rows, vocab));
    if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
    const Plan p = plan_scan(dtype, false, rows, vocab);
    ScanArgs a = scan_args(logits, dtype, rows, vocab, ld, p, 1.0);
    a.out_idx = out_token;
    a.tickets = at<uint32_t>(ws, w.tickets);
    a.p_key = at<uint64_t>(ws, w.p_key);
    a.p_m = at<float>(ws, w.p_m);
    a.p_s = at<double>(ws, w.p_s);
    a.out_logp0 = out_logprob;
    return launched(launch_scan(dtype, false, a, s));
  }

  if (top_k == 0) {
    if (vocab > kMaxDrawVocab) return VSEL_EINVAL;
    Layout L;
    const RowDrawWs w = rowdraw_layout(L, rows, vocab, plan_scan_bound(rows, vocab));
    if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
    const Plan ps = plan_scan(dtype, false, rows, vocab);
    const Plan pd = plan_draw(rows, vocab, resident_scan(dtype, false));
    ScanArgs a = scan_args(logits, dtype, rows, vocab, ld, ps, temperature);
    a.tickets = at<uint32_t>(ws, w.scan.tickets);
    a.p_key = at<uint64_t>(ws, w.scan.p_key);
    a.p_m = at<float>(ws, w.scan.p_m);
    a.p_s = at<double>(ws, w.scan.p_s);
    a.st_amax = at<uint32_t>(ws, w.st.amax);
    a.st_max = at<float>(ws, w.st.mx);
    a.st_bad = at<uint32_t>(ws, w.st.bad);
    if (scan_moments) {
      a.m_n = at<double>(ws, cw->mom.p_n);
      a.m_mean = at<double>(ws, cw->mom.p_mean);
      a.m_m2 = at<double>(ws, cw->mom.p_m2);
      a.sigma = at<double>(ws, cw->mom.sigma);
      sigma = a.sigma;
    }
    hipError_t e = launch_scan(dtype, false, a, s);
    if (e != hipSuccess) return VSEL_EDEVICE;
    if (typical_p < 1.0f || top_p < 1.0f) {
      // typical-p over the whole row (then top-p, min-p, the draw), or the
      // nucleus over the whole row (then min-p, the draw in value order)
      NucArgs n{};
      n.x = logits;
      n.ld = ld;
      n.rows = rows;
      n.V = vocab;
      n.st_max = a.st_max;
      n.st_bad = a.st_bad;
      n.sigma = sigma;
      n.top_n_sigma = top_n_sigma;
      n.top_p = top_p;
      n.min_p = min_p;
      n.typical_p = typical_p;
      n.T = temperature;
      n.u = u;
      n.out_token = out_token;
      n.out_logp = out_logprob;
      const Plan pn = plan_nucleus(rows, vocab);
      n.seg_len = pn.seg_len;
      n.S = pn.S;
      n.vec = a.vec1;
      const NucWs& nw = cw->nuc;
      n.tickets = at<uint32_t>(ws, nw.tickets);
      n.h0w = at<double>(ws, nw.h0w);
      n.h0c = at<uint32_t>(ws, nw.h0c);
      n.hTw = at<double>(ws, nw.hTw);
      n.hTc = at<uint32_t>(ws, nw.hTc);
      n.lkey = at<uint64_t>(ws, nw.lkey);
      n.lbits = at<uint32_t>(ws, nw.lbits);
      n.lcnt = at<uint32_t>(ws, nw.lcnt);
      n.gcnt = at<uint32_t>(ws, nw.gcnt);
      n.gbits = at<uint32_t>(ws, nw.gbits);
      n.gidx = at<uint32_t>(ws, nw.gidx);
      n.p_z0 = at<double>(ws, nw.p_z0);
      n.p_a = at<double>(ws, nw.p_a);
      n.p_at = at<double>(ws, nw.p_at);
      n.p_a2 = at<double>(ws, nw.p_a2);
      n.plan = at<NucPlan>(ws, nw.plan);
      n.jobs = at<SelJob>(ws, nw.jobs);
      return launched(typical_p < 1.0f ? launch_row_typical(dtype, n, s) : launch_row_nucleus(dtype, n, s));
    }
    DrawArgs d{};
    d.x = logits;
    d.ld = ld;
    d.rows = rows;
    d.V = vocab;
    d.seg_len = pd.seg_len;
    d.S = pd.S;
    d.vec = a.vec1;
    d.T = temperature;
    d.u = u;
    d.st_max = a.st_max;
    d.st_bad = a.st_bad;
    d.out_token = out_token;
    d.out_logp = out_logprob;
    d.tickets = at<uint32_t>(ws, w.dtickets);
    d.nchunk = cdiv(vocab, kChunk);
    d.p_w = at<double>(ws, w.p_w);
    d.p_c = at<double>(ws, w.p_c);
    d.top_n_sigma = top_n_sigma;
    d.min_p = min_p;
    d.sigma = sigma;
    return launched(launch_draw_rows(dtype, d, s));
  }

  const int32_t k = (int32_t)std::min<int64_t>(top_k, vocab);
  TopkArgs a{};
  a.mode = 1;
  a.temperature = temperature;
  a.top_p = top_p;
  a.top_n_sigma = top_n_sigma;
  a.typical_p = typical_p;
  a.min_p = min_p;
  a.sigma = sigma;
  if (fused_moments) {
    a.m_n = at<double>(ws, cw->mom.p_n);
    a.m_mean = at<double>(ws, cw->mom.p_mean);
    a.m_m2 = at<double>(ws, cw->mom.p_m2);
  }
  a.u = u;
  a.out_token = out_token;
  a.out_logp = out_logprob;
  return topk_common(logits, dtype, rows, vocab, ld, k, false, a, ws, ws_bytes, stream);
}

// The sampler is the chain with top_k and top_p only (its workspace has the
// chain's layout, so top_k == 0 with top_p < 1 takes the whole-row nucleus).
vsel_status vsel_sample(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                        float temperature, int32_t top_k, float top_p, const float* u, uint32_t* out_token,
                        float* out_logprob, void* ws, size_t ws_bytes, void* stream) {
  return vsel_sample_chain(logits, dtype, rows, vocab, ld, temperature, 0.0f, top_k, 1.0f, top_p, 0.0f, u, out_token,
                           out_logprob, ws, ws_bytes, stream);
}

vsel_status vsel_sample_chain(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                              float temperature, float top_n_sigma, int32_t top_k, float typical_p, float top_p,
                              float min_p, const float* u, uint32_t* out_token, float* out_logprob, void* ws,
                              size_t ws_bytes, void* stream) {
  // everything sample_impl checks, before the moments pass can launch
  if (!logits || !u || !out_token || !elem_ok(dtype) || !rows_ok(rows, vocab, ld) ||
      !aligned_elem(logits, elem_size(dtype)))
    return VSEL_EINVAL;
  if (!(temperature >= 0.0f) || std::isinf(temperature) || !(top_k >= 0 && top_k <= VSEL_K_MAX) ||
      !(top_p > 0.0f && top_p <= 1.0f) || !(top_n_sigma >= 0.0f) || std::isinf(top_n_sigma) ||
      !(typical_p > 0.0f && typical_p <= 1.0f) || !(min_p >= 0.0f && min_p <= 1.0f))
    return VSEL_EINVAL;
  const size_t base = sample_ws_bytes(rows, vocab, top_k);
  if (base == 0) return VSEL_EINVAL;
  Layout L;
  L.off = align_up(base);
  const ChainWs cw = chain_layout(L, rows, vocab, top_k);
  if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
  return sample_impl(logits, dtype, rows, vocab, ld, temperature, top_k, top_p, top_n_sigma, typical_p, min_p, &cw,
                     u, out_token, out_logprob, ws, ws_bytes, stream);
}

// Argument checks, pass 1 (row statistics of every target and draft row)
// and the common kernel arguments of the speculative entry points.
// fused_draw: the draws will run in pass 2's launch (modified rejection
// sampling at T > 0), which sets their segments.
static vsel_status spec_prepare(const float* target, int64_t ld_t, const float* draft, int64_t ld_d, int64_t batch,
                                int32_t gamma, int64_t vocab, float temperature, const uint32_t* draft_tokens,
                                void* ws, size_t ws_bytes, hipStream_t s, SpecArgs& p, bool fused_draw = false) {
  if (!target || !draft || !draft_tokens) return VSEL_EINVAL;
  if (batch < 1 || gamma < 1 || gamma > kMaxSegments || vocab < 1 || vocab >= (int64_t(1) << 31) || ld_t < vocab ||
      ld_d < vocab)
    return VSEL_EINVAL;
  if (!rows_ok(batch * (2 * (int64_t)gamma + 1), vocab, vocab)) return VSEL_EINVAL;
  if (!(temperature >= 0.0f) || std::isinf(temperature)) return VSEL_EINVAL;
  if (!aligned_elem(target, 4) || !aligned_elem(draft, 4) || vocab > kMaxDrawVocab) return VSEL_EINVAL;
  const int64_t B = batch, G = gamma;
  Layout L;
  const SpecWs w = spec_layout(L, B, G, vocab, plan_scan_bound(B * (2 * G + 1), vocab), plan_scan_bound(B * G, vocab));
  if (!ws_ok(ws, ws_bytes, L.off)) return VSEL_EWORKSPACE;
  const Plan ps = plan_scan(VSEL_F32, temperature > 0.0f, B * (2 * G + 1), vocab);
  const Plan pp = plan_scan(VSEL_F32, true, B * G, vocab, 2);  // the position passes read two rows

  ScanArgs a = scan_args(target, VSEL_F32, B * (G + 1), vocab, ld_t, ps, temperature);
  a.x2 = draft;
  a.ld2 = ld_d;
  a.rows2 = B * G;
  a.vec2 = aligned16(draft, ld_d, 4) ? 1 : 0;
  a.tickets = at<uint32_t>(ws, w.scan.tickets);
  a.p_key = at<uint64_t>(ws, w.scan.p_key);
  a.p_m = at<float>(ws, w.scan.p_m);
  a.p_s = at<double>(ws, w.scan.p_s);
  a.st_amax = at<uint32_t>(ws, w.st.amax);
  a.st_max = at<float>(ws, w.st.mx);
  a.st_lse = at<double>(ws, w.st.lse);
  a.st_bad = at<uint32_t>(ws, w.st.bad);
  if (launch_scan(VSEL_F32, temperature > 0.0f, a, s) != hipSuccess) return VSEL_EDEVICE;

  p = SpecArgs{};
  p.tgt = target;
  p.dft = draft;
  p.ld_t = ld_t;
  p.ld_d = ld_d;
  p.B = B;
  p.gamma = gamma;
  p.V = vocab;
  p.T = temperature;
  p.inv_T = temperature > 0 ? 1.0f / temperature : 0.0f;
  p.lse_c = a.lse_c;
  p.tokens = draft_tokens;
  p.seg_len = pp.seg_len;
  p.S = pp.S;
  p.vec_t = a.vec1;
  p.vec_d = a.vec2;
  p.st_amax = a.st_amax;
  p.st_max = a.st_max;
  p.st_lse = a.st_lse;
  p.st_bad = a.st_bad;
  p.tk_pos = at<uint32_t>(ws, w.tk_pos);
  p.tk_seq = at<uint32_t>(ws, w.tk_seq);
  p.tk_draw = at<uint32_t>(ws, w.tk_draw);
  p.p_summin = at<double>(ws, w.p_summin);
  p.acc = at<uint32_t>(ws, w.acc);
  p.draw_L = at<int32_t>(ws, w.draw_L);
  p.p_lse = at<double>(ws, w.p_lse);
  const Plan pd = fused_draw ? plan_draw_fused(B, vocab) : plan_draw(B, vocab, resident_scan(VSEL_F32, true));
  p.dseg = pd.seg_len;
  p.dS = pd.S;
  p.nchunk = cdiv(vocab, kChunk);
  p.p_w = at<double>(ws, w.p_w);
  p.p_c = at<double>(ws, w.p_c);
  p.p_cb = at<double>(ws, w.p_cb);
  p.p_cf = at<uint32_t>(ws, w.p_cf);
  p.p_low = at<double>(ws, w.p_low);
  p.p_wt = at<double>(ws, w.p_wt);
  return VSEL_OK;
}

vsel_status vsel_spec_accept(const float* target, int64_t ld_t, const float* draft, int64_t ld_d, int64_t batch,
                             int32_t gamma, int64_t vocab, float temperature, const uint32_t* draft_tokens,
                             const float* u_accept, const float* u_resid, const float* u_bonus,
                             int32_t* out_len_mrs, uint32_t* out_tok_mrs, int32_t* out_len_aa,
                             uint32_t* out_tok_aa, float* out_summin, float* out_sumprod, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!u_accept || !u_resid || !u_bonus || !out_len_mrs || !out_tok_mrs) return VSEL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  SpecArgs p;
  const vsel_status st = spec_prepare(target, ld_t, draft, ld_d, batch, gamma, vocab, temperature, draft_tokens, ws,
                                      ws_bytes, s, p, temperature > 0.0f);
  if (st != VSEL_OK) return st;
  p.u_acc = u_accept;
  p.u_res = u_resid;
  p.u_bon = u_bonus;
  p.len_mrs = out_len_mrs;
  p.tok_mrs = out_tok_mrs;
  p.len_aa = out_len_aa;
  p.tok_aa = out_tok_aa;
  p.summin = out_summin;
  p.sumprod = out_sumprod;
  return launched(launch_spec(p, s));
}

// The filter pass of filtered speculative acceptance: for the target rows and
// then the draft rows, the smallest kept key and the kept set's lse at T.
// top_k >= 1: the top-k kernel's candidates (top-p and min-p on them);
// top_k == 0: the whole-row nucleus (top_p < 1) or the min-p threshold.
// Temperature 0 or no filter: nothing to do (the unfiltered rules).
static vsel_status spec_filter(SpecArgs& p, int32_t top_k, float top_p, float min_p, void* ws, const SpecFiltWs& fw,
                               hipStream_t s) {
  if (p.T == 0.0f || (top_k == 0 && top_p >= 1.0f && min_p <= 0.0f)) return VSEL_OK;
  const int64_t G = p.gamma, nT = p.B * (G + 1), nD = p.B * G;
  uint64_t* kfl = at<uint64_t>(ws, fw.kfl);
  double* lse = at<double>(ws, fw.lse);
  if (top_k >= 1) {  // the top-k passes, per part
    for (int part = 0; part < 2; ++part) {
      const float* x = part == 0 ? p.tgt : p.dft;
      const int64_t ld = part == 0 ? p.ld_t : p.ld_d;
      const int64_t rows = part == 0 ? nT : nD, off = part == 0 ? 0 : nT;
      TopkArgs a{};
      a.mode = 2;
      a.temperature = p.T;
      a.top_p = top_p;
      a.top_n_sigma = 0.0f;
      a.typical_p = 1.0f;
      a.min_p = min_p;
      a.out_kfl = kfl + off;
      a.out_lse_f = lse + off;
      const int32_t k = (int32_t)std::min<int64_t>(top_k, p.V);
      const vsel_status st =
          topk_common(x, VSEL_F32, rows, p.V, ld, k, false, a, at<char>(ws, fw.sub_topk), fw.topk_bytes, s);
      if (st != VSEL_OK) return st;
    }
  } else {  // the whole-row passes over the target rows and then the draft rows, in one set of launches
    void* sub = at<char>(ws, fw.sub_nuc);
    const int64_t rows = nT + nD;
    Layout L;
    const NucWs nw = nucleus_layout(L, rows, plan_scan_bound(rows, p.V));
    NucArgs n{};
    n.x = p.tgt;
    n.ld = p.ld_t;
    n.x2 = p.dft;
    n.ld2 = p.ld_d;
    n.rows1 = nT;
    n.rows = rows;
    n.V = p.V;
    n.vec = aligned16(p.tgt, p.ld_t, 4) && aligned16(p.dft, p.ld_d, 4) ? 1 : 0;
    n.st_max = p.st_max;
    n.st_bad = p.st_bad;
    n.sigma = nullptr;
    n.top_n_sigma = 0.0f;
    n.top_p = top_p;
    n.min_p = min_p;
    n.T = p.T;
    n.tickets = at<uint32_t>(sub, nw.tickets);
    n.h0w = at<double>(sub, nw.h0w);
    n.h0c = at<uint32_t>(sub, nw.h0c);
    n.hTw = at<double>(sub, nw.hTw);
    n.hTc = at<uint32_t>(sub, nw.hTc);
    n.lkey = at<uint64_t>(sub, nw.lkey);
    n.lbits = at<uint32_t>(sub, nw.lbits);
    n.lcnt = at<uint32_t>(sub, nw.lcnt);
    n.gcnt = at<uint32_t>(sub, nw.gcnt);
    n.gbits = at<uint32_t>(sub, nw.gbits);
    n.gidx = at<uint32_t>(sub, nw.gidx);
    n.p_z0 = at<double>(sub, nw.p_z0);
    n.p_a = at<double>(sub, nw.p_a);
    n.p_at = at<double>(sub, nw.p_at);
    n.p_a2 = at<double>(sub, nw.p_a2);
    n.plan = at<NucPlan>(sub, nw.plan);
    n.out_kfl = kfl;
    n.out_lse_f = lse;
    if (top_p < 1.0f) {
      const Plan pn = plan_nucleus(rows, p.V);
      n.seg_len = pn.seg_len;
      n.S = pn.S;
      if (launch_row_nucleus(VSEL_F32, n, s) != hipSuccess) return VSEL_EDEVICE;
    } else {
      const Plan ps = plan_scan(VSEL_F32, false, rows, p.V);
      n.seg_len = ps.seg_len;
      n.S = ps.S;
      if (launch_kept_lse(VSEL_F32, n, s) != hipSuccess) return VSEL_EDEVICE;
    }
  }
  p.kfl = kfl;
  p.st_lse = lse;
  return VSEL_OK;
}

static bool filters_ok(int32_t top_k, float top_p, float min_p) {
  return top_k >= 0 && top_k <= VSEL_K_MAX && top_p > 0.0f && top_p <= 1.0f && min_p >= 0.0f && min_p <= 1.0f;
}

// The whole workspace of a filtered call, checked before anything launches.
static bool spec_filtered_ws(int64_t batch, int32_t gamma, int64_t vocab, void* ws, size_t ws_bytes, SpecFiltWs& fw) {
  if (batch < 1 || gamma < 1 || gamma > kMaxSegments || vocab < 1 || vocab > kMaxDrawVocab ||
      !rows_ok(batch * (2 * (int64_t)gamma + 1), vocab, vocab))
    return true;  // spec_prepare reports the bad argument
  Layout L;
  spec_layout(L, batch, gamma, vocab, plan_scan_bound(batch * (2 * (int64_t)gamma + 1), vocab),
              plan_scan_bound(batch * (int64_t)gamma, vocab));
  fw = spec_filter_layout(L.off, batch, gamma, vocab);
  return ws_ok(ws, ws_bytes, fw.end);
}

vsel_status vsel_spec_accept_filtered(const float* target, int64_t ld_t, const float* draft, int64_t ld_d,
                                      int64_t batch, int32_t gamma, int64_t vocab, float temperature, int32_t top_k,
                                      float top_p, float min_p, const uint32_t* draft_tokens, const float* u_accept,
                                      const float* u_resid, const float* u_bonus, int32_t* out_len_mrs,
                                      uint32_t* out_tok_mrs, int32_t* out_len_aa, uint32_t* out_tok_aa,
                                      float* out_summin, float* out_sumprod, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!u_accept || !u_resid || !u_bonus || !out_len_mrs || !out_tok_mrs) return VSEL_EINVAL;
  if (!filters_ok(top_k, top_p, min_p)) return VSEL_EINVAL;
  SpecFiltWs fw{};
  if (!spec_filtered_ws(batch, gamma, vocab, ws, ws_bytes, fw)) return VSEL_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  SpecArgs p;
  vsel_status st = spec_prepare(target, ld_t, draft, ld_d, batch, gamma, vocab, temperature, draft_tokens, ws,
                                ws_bytes, s, p, temperature > 0.0f);
  if (st != VSEL_OK) return st;
  if ((st = spec_filter(p, top_k, top_p, min_p, ws, fw, s)) != VSEL_OK) return st;
  p.u_acc = u_accept;
  p.u_res = u_resid;
  p.u_bon = u_bonus;
  p.len_mrs = out_len_mrs;
  p.tok_mrs = out_tok_mrs;
  p.len_aa = out_len_aa;
  p.tok_aa = out_tok_aa;
  p.summin = out_summin;
  p.sumprod = out_sumprod;
  return launched(launch_spec(p, s));
}

vsel_status vsel_spec_match_filtered(const float* target, int64_t ld_t, const float* draft, int64_t ld_d,
                                     int64_t batch, int32_t gamma, int64_t vocab, float temperature, int32_t top_k,
                                     float top_p, float min_p, const uint32_t* draft_tokens, const float* u_match,
                                     int32_t* out_len, uint32_t* out_tok, float* out_sumprod, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!u_match || !out_len || !out_tok) return VSEL_EINVAL;
  if (!filters_ok(top_k, top_p, min_p)) return VSEL_EINVAL;
  SpecFiltWs fw{};
  if (!spec_filtered_ws(batch, gamma, vocab, ws, ws_bytes, fw)) return VSEL_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  SpecArgs p;
  vsel_status st =
      spec_prepare(target, ld_t, draft, ld_d, batch, gamma, vocab, temperature, draft_tokens, ws, ws_bytes, s, p);
  if (st != VSEL_OK) return st;
  if ((st = spec_filter(p, top_k, top_p, min_p, ws, fw, s)) != VSEL_OK) return st;
  p.match = 1;
  p.u_match = u_match;
  p.len_sm = out_len;
  p.tok_sm = out_tok;
  p.sumprod = out_sumprod;
  return launched(launch_spec_match(p, s));
}

vsel_status vsel_spec_match(const float* target, int64_t ld_t, const float* draft, int64_t ld_d, int64_t batch,
                            int32_t gamma, int64_t vocab, float temperature, const uint32_t* draft_tokens,
                            const float* u_match, int32_t* out_len, uint32_t* out_tok, float* out_sumprod,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!u_match || !out_len || !out_tok) return VSEL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  SpecArgs p;
  const vsel_status st =
      spec_prepare(target, ld_t, draft, ld_d, batch, gamma, vocab, temperature, draft_tokens, ws, ws_bytes, s, p);
  if (st != VSEL_OK) return st;
  p.match = 1;
  p.u_match = u_match;
  p.len_sm = out_len;
  p.tok_sm = out_tok;
  p.sumprod = out_sumprod;
  return launched(launch_spec_match(p, s));
}

}  // extern "C"

namespace vsel {

int topk_entry(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k, float* out_vals,
               uint32_t* out_ids, uint32_t* out_argmax, float* out_lse, void* ws, size_t ws_bytes, void* stream,
               bool exact_layout) {
  if (!logits || !out_vals || !out_ids || !elem_ok(dtype) || !rows_ok(rows, vocab, ld) ||
      !aligned_elem(logits, elem_size(dtype)) || k < 1 || k > VSEL_K_MAX || k > vocab)
    return VSEL_EINVAL;
  TopkArgs a{};
  a.mode = 0;
  a.out_vals = out_vals;
  a.out_ids = out_ids;
  a.out_argmax = out_argmax;
  a.out_lse = out_lse;
  return topk_common(logits, dtype, rows, vocab, ld, k, out_lse != nullptr, a, ws, ws_bytes, stream, exact_layout);
}

}  // namespace vsel
