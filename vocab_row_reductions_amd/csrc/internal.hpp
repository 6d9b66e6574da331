// internal.hpp -- kernel argument blocks and launcher entry points of the
// vsel library (not part of the public C ABI in include/vsel.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vsel {

constexpr size_t kWsAlign = 256;
constexpr int kCapSmall = 2048;  // LDS candidate records per workgroup (about 35 KiB of LDS in all)
constexpr int kCapLarge = 4096;  // for large k or many segments per row
constexpr int kMaxSegments = 256;  // segments per row, at most (one thread each in a merge)
constexpr int kTopkGroups = 8;       // 16-byte groups per lane per top-k tile
constexpr int kChunk = 256;          // draw chunk: elements per float64 chunk mass (one per thread)
constexpr int kChunksPerSeg = 1024;  // chunks per draw segment, at most

inline size_t align_up(size_t x, size_t a = kWsAlign) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- row scan
// One pass over each row: first-maximum argmax, the maximum value, the
// latch for nonfinite rows and (optionally) log-sum-exp at temperature T.
// Rows [0, rows1) come from x1 (stride ld1), rows [rows1, rows1+rows2) from x2.
struct ScanArgs {
  const void* x1;
  const void* x2;
  int64_t ld1, ld2;
  int64_t rows1, rows2;
  int64_t V;
  int64_t seg_len;     // elements per segment, a multiple of 8
  int32_t S;           // segments per row
  int32_t vec1, vec2;  // 16-byte aligned rows
  float lse_c;         // log2(e) / T
  double T;            // temperature of the log-sum-exp
  // user outputs (argmax op)
  uint32_t* out_idx;
  float* out_val;
  float* out_logp0;    // greedy sampling: 0, or NaN for a fail-closed row
  // row-stat outputs (spec / sample), any may be null
  uint32_t* st_amax;
  float* st_max;
  double* st_lse;
  uint32_t* st_bad;
  // workspace
  uint32_t* tickets;
  uint64_t* p_key;
  float* p_m;
  double* p_s;
  // greedy serving variant: ids taken as -inf inside the reduction, and a
  // per-row status (0 ok, 1 nonfinite, 2 no element above -inf)
  const uint32_t* excl;
  int32_t n_excl;      // 0 .. kMaxExcluded
  uint32_t* out_status;
  // row moments in the same pass (the sampler chain's top-n-sigma over whole
  // rows; no log-sum-exp, no excluded ids): per (row, segment) count, mean
  // and squared deviations of the values above -inf, and each row's
  // standard deviation (null: no moments)
  double* m_n;
  double* m_mean;
  double* m_m2;
  double* sigma;
};
constexpr int kMaxExcluded = 256;

// ---------------------------------------------------------------- top-k
struct TopkArgs {
  const void* x;
  int64_t ld;
  int64_t rows;
  int64_t V;
  int64_t seg_len;
  int32_t S;
  int32_t k;
  int32_t vec;
  int32_t mode;   // 0: top-k outputs, 1: sampling tail, 2: kept-set floor and lse
  float* out_vals;
  uint32_t* out_ids;
  uint32_t* out_argmax;
  float* out_lse;
  // sampling: the ordered chain (ChainParams in device.hpp)
  float temperature;
  float top_p;
  float top_n_sigma;    // 0: off
  float typical_p;      // 1: off (needs k <= kWaveTopkMax)
  float min_p;          // 0: off
  const double* sigma;  // [rows] standard deviation of each row (top_n_sigma > 0)
  // or (per-wave kernel) the row moments taken in the same pass: per
  // (row, segment) count, mean and squared deviations of the values above
  // -inf (non-null: the kernel computes sigma itself)
  double* m_n;
  double* m_mean;
  double* m_m2;
  // mode 2 (filtered speculative acceptance): per row, the smallest kept
  // composite key and the kept set's log sum of exp(z/T); nothing is drawn
  uint64_t* out_kfl;
  double* out_lse_f;
  const float* u;
  uint32_t* out_token;
  float* out_logp;
  // workspace (used when S > 1)
  uint32_t* tickets;
  uint64_t* rec_key;
  uint32_t* rec_bits;
  uint32_t* rec_cnt;
  float* p_m;
  double* p_s;
};

// ---------------------------------------------------------------- speculative acceptance
struct SpecArgs {
  const float* tgt;
  const float* dft;
  int64_t ld_t, ld_d;
  int64_t B;
  int32_t gamma;
  int64_t V;
  float T;
  float inv_T;
  float lse_c;
  const uint32_t* tokens;
  const float* u_acc;
  const float* u_res;
  const float* u_bon;
  int32_t* len_mrs;
  uint32_t* tok_mrs;
  int32_t* len_aa;
  uint32_t* tok_aa;
  float* summin;
  int64_t seg_len;
  int32_t S;
  int32_t vec_t, vec_d;
  // row stats from the scan pass: target rows then draft rows
  const uint32_t* st_amax;
  const float* st_max;
  const double* st_lse;
  const uint32_t* st_bad;
  // workspace
  uint32_t* tk_pos;     // [B*gamma] per-position tickets
  uint32_t* tk_seq;     // [B]       per-sequence tickets
  uint32_t* tk_draw;    // [B]       per-sequence draw tickets
  double* p_summin;     // [B*gamma*S]
  uint32_t* acc;        // [B*gamma]
  int32_t* draw_L;      // [B]: -1 none, 0..gamma-1 residual at L, gamma bonus
  double* p_lse;        // [B*2*dS] residual draw: the segments' float64 sums of P, then of Q
  // the draw: segments of dseg elements (a multiple of kChunk), dS per row
  int64_t dseg;
  int32_t dS;
  int64_t nchunk;       // chunks per row, ceil(V / kChunk)
  double* p_w;          // [B*dS] segment masses
  double* p_c;          // [B*nchunk] chunk masses
  double* p_cb;         // [B*nchunk] residual draw: the draft row's part of each chunk
  uint32_t* p_cf;       // [B*nchunk] residual draw: chunks to recompute element by element
  // sampler-match (vsel_spec_match): a fresh draw from p at each position
  int32_t match;
  const float* u_match;  // [B*(gamma+1)]
  int32_t* len_sm;
  uint32_t* tok_sm;
  float* sumprod;        // [B*gamma] or null
  double* p_low;         // [B*gamma*S] mass of p below the drafted token, per segment
  double* p_wt;          // [B*gamma*S] mass of p, per segment
  // filtered p and q (top-k / top-p / min-p): element x of a row is kept iff
  // its composite key is >= kfl[row] (target rows then draft rows); st_lse
  // then holds log sum over the kept elements of exp(z/T), exact in float64.
  const uint64_t* kfl;   // null: unfiltered
};

// Plain full-row draw for vsel_sample with top_k == 0.
struct DrawArgs {
  const void* x;
  int64_t ld;
  int64_t rows;
  int64_t V;
  int64_t seg_len;
  int32_t S;
  int32_t vec;
  float T;
  const float* u;
  const float* st_max;
  const uint32_t* st_bad;
  uint32_t* out_token;
  float* out_logp;
  uint32_t* tickets;
  int64_t nchunk;       // chunks per row, ceil(V / kChunk); seg_len is a multiple of kChunk
  double* p_w;          // [rows*S] segment masses
  double* p_c;          // [rows*nchunk] chunk masses
  // the chain's threshold filters over the whole row: elements below
  // st_max - top_n_sigma * sigma or st_max + log(min_p) weigh nothing
  float top_n_sigma;    // 0: off
  float min_p;          // 0: off
  const double* sigma;  // [rows]
};

// Mean and standard deviation of each row's values above -inf (float64,
// shifted sums merged in a fixed order), for the top-n-sigma filter.
struct MomArgs {
  const void* x;
  int32_t vec;          // rows start and stride 16-byte aligned (segments are multiples of 8 elements)
  int64_t ld;
  int64_t rows;
  int64_t V;
  int64_t seg_len;
  int32_t S;
  uint32_t* tickets;
  double* p_n;          // [rows*S] segment partials: count, mean, sum of squared deviations
  double* p_mean;
  double* p_m2;
  double* sigma;        // [rows] output
};

// The sampler chain over whole rows with a top-p cut: three passes over
// (row, segment) workgroups (a guide histogram, the cut window, the draw
// window) and a one-workgroup fallback.  Histograms, window counters and
// tickets are zero between calls.
constexpr int kNucBins = 4096;     // guide bins per row
constexpr int kNucCap = 4096;      // window candidates per row
constexpr int kGatherCap = 2048;   // gathered candidates per (row, segment)
struct NucPlan {                   // per row, written by the last workgroup of a pass
  uint32_t state;                  // 0 cut placed, 1 draw pass needed, 2 done, 3/4 row/draw left to one workgroup
  uint32_t b_lo, b_hi;             // cut window (untempered guide bins)
  uint32_t c_lo, c_hi;             // draw window (tempered guide bins, above the cut window)
  uint32_t listed;                 // 1: every candidate the later passes reach is in the gathered list
  uint32_t h0top, hTtop;           // highest non-empty bins (short of the last) of the row's two histograms
  double z0;                       // exact candidate mass, untempered
  double a_above;                  // exact untempered mass of the candidates above the cut window
  double wt;                       // exact kept mass, tempered
  uint64_t kfin;                   // smallest kept composite key
};
// One row's weighted selection, carried from pass to pass of typical-p over
// whole rows (the typical cut, then top-p within the typical set, then the
// draw): the candidate set and order, the target, and the results.
struct SelJob {
  double m, thr, T;      // candidates z > -inf, z >= thr; weights exp((z - m) / T)
  double c, span;        // the typical centre; the bins' span (value order: of (m - z) / T, typical: of |z - c|)
  double span_all;       // typical order: the span of every candidate's distance
  double frac;           // target: the first candidate whose cumulative weight reaches frac x total
  uint64_t kfloor, kT;   // order-key floor; typical-set floor on the score key (0: none)
  int32_t order, strict; // 0 value, 1 typicality; strict: cumulative weight must pass the target
  int32_t state;         // 0 none, 1 guide pass due, 2 window pass due, 3 left to one workgroup, 4 selected
  int32_t step;          // 1 typical cut, 2 top-p within the set, 3 the draw
  uint32_t b_lo, b_hi;   // window (guide bins)
  uint32_t bits;         // selected candidate's element bits
  uint32_t listed;       // 1: every candidate of this and the later selections is in the gathered list
  uint32_t htop, pad;    // highest non-empty bin (short of the last) of the row's histogram
  uint64_t key;          // selected candidate's order key
  double tot;            // exact total weight of the candidates
  double tot_known;      // > 0: that total, known before the guide pass (no exact sums there)
  double cum;            // exact cumulative weight through the selected candidate
  double zmax;           // largest value among the candidates up to the selected one
  double aux;            // the typical set's largest value (the min_p reference)
};
struct NucArgs {
  const void* x;
  int64_t ld;
  // rows1 > 0 and x2: rows from rows1 on are rows of x2 (stride ld2), so
  // that two batches (speculative target and draft rows) run in one launch
  const void* x2;
  int64_t ld2, rows1;
  int64_t rows;
  int64_t V;
  int64_t seg_len;         // a multiple of 8 elements
  int32_t S;
  int32_t vec;             // rows start and stride 16-byte aligned (both batches)
  const float* st_max;     // [rows] row maxima (scan)
  const uint32_t* st_bad;  // [rows] fail-closed rows (scan)
  const double* sigma;     // [rows] standard deviations (top_n_sigma > 0)
  float top_n_sigma, top_p, min_p, T;
  float typical_p;         // (typical-p over whole rows)
  const float* u;
  uint32_t* out_token;
  float* out_logp;
  uint32_t* tickets;       // [rows*3]
  double* h0w;             // [rows*kNucBins] untempered guide masses
  uint32_t* h0c;           // [rows*kNucBins] counts
  double* hTw;             // [rows*kNucBins] tempered guide masses (above the cut window)
  uint32_t* hTc;
  uint64_t* lkey;          // [rows*kNucCap] window candidates
  uint32_t* lbits;
  uint32_t* lcnt;          // [rows]
  // candidates the first guide pass gathered (those within the crossing
  // bound), per (row, segment) slot in stream order: count (kGatherCap + 1:
  // overflowed), element bits and indices
  uint32_t* gcnt;          // [rows*S]
  uint32_t* gbits;         // [rows*S*kGatherCap]
  uint32_t* gidx;
  double* p_z0;            // [rows*S] segment partials
  double* p_a;
  double* p_at;
  double* p_a2;
  NucPlan* plan;           // [rows]
  SelJob* jobs;            // [rows] (typical-p)
  // floor mode (filtered speculative acceptance): instead of drawing, the
  // kept set's smallest composite key and log sum of exp(z/T) over it
  uint64_t* out_kfl;       // null: sampling
  double* out_lse_f;
};

hipError_t launch_scan(int dtype, bool want_lse, const ScanArgs& a, hipStream_t s);
hipError_t launch_topk(int dtype, bool want_lse, int cap, const TopkArgs& a, hipStream_t s);
// Per-wave filtering variant of the top-k kernel: k <= kWaveTopkMax, rows
// whose start and stride are 16-byte aligned, merge buffer of kCapSmall.
constexpr int kWaveTopkMax = 128;
hipError_t launch_topk_wave(int dtype, bool want_lse, const TopkArgs& a, hipStream_t s);
int topk_wave_blocks_per_cu(int dtype, bool want_lse);
// Workgroups of a kernel variant that fit on one CU at once (0 if unknown).
int scan_blocks_per_cu(int dtype, bool want_lse);
int topk_blocks_per_cu(int dtype, bool want_lse, int cap);
hipError_t launch_spec(const SpecArgs& a, hipStream_t s);
hipError_t launch_spec_match(const SpecArgs& a, hipStream_t s);
hipError_t launch_draw_rows(int dtype, const DrawArgs& a, hipStream_t s);
hipError_t launch_moments(int dtype, const MomArgs& a, hipStream_t s);
hipError_t launch_row_nucleus(int dtype, const NucArgs& a, hipStream_t s);
// Floor mode with min_p only (top_p == 1): kept = z >= max + log(min_p).
// Uses x, ld, rows, V, seg_len, S, vec, st_max, st_bad, min_p, T, tickets,
// p_z0 and the outputs.
hipError_t launch_kept_lse(int dtype, const NucArgs& a, hipStream_t s);
// Typical-p over whole rows, then top-p, min-p and the draw, in passes over
// (row, segment) workgroups (the nucleus arguments, typical_p and jobs).
hipError_t launch_row_typical(int dtype, const NucArgs& a, hipStream_t s);

// vsel_topk's argument checks, layout and launch, returning a vsel_status.
// exact_layout places the workspace for the call's own segment plan instead of
// the shape's bound; the ticket counters lead the layout either way, in
// max(64 KiB, 4 x rows) bytes.
int topk_entry(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k, float* out_vals,
               uint32_t* out_ids, uint32_t* out_argmax, float* out_lse, void* ws, size_t ws_bytes, void* stream,
               bool exact_layout);

}  // namespace vsel
