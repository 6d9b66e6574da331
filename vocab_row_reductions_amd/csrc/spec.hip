// spec.hip -- speculative-decoding acceptance on the device, and the
// full-row categorical draw.
//
// Modified rejection sampling ("speculative-acceptance.md", "Modified
// rejection sampling"; the exact CPU acceptance of "Chapter 21", section
// 21.9) needs, per verified position, two full-vocabulary reductions (the
// pages' MLX version pays them as extra passes plus a host sync per
// position).  Here the whole batch runs in two launches on one stream and
// nothing returns to the host:
//   1. row scan (scan.hip) over all target and draft rows: argmax, maximum,
//      latch, log-sum-exp at T;
//   2. coupling pass, one workgroup per (position, segment): p = exp(z/T -
//      lse_p), q = exp(d/T - lse_q), sum of min(p, q) (the acceptance ceiling
//      of "The acceptance ceiling").  The last workgroup of a position decides
//      u * q(t) <= p(t) in float64; the last position of a sequence finds the
//      first rejection L for both rules and writes every emitted token except
//      the draw;
//   and in the same launch, the draw: the accept tests need only pass 1's
//   log-sum-exps, so the draw's workgroups find L themselves and run beside
//   the coupling pass.  They take float64 masses of each segment of the draw
//   row (residual max(p - q, 0), or p for the bonus token), then the last
//   one picks the segment whose prefix crosses u * W and rescans it in id
//   order.  The residual mixes p and q, so both need float64 log-sum-exps:
//   the same pass sums them and the residual's parts of each chunk (see
//   resid_chunks), and the last workgroup combines them.
// The filtered rules run the filter passes between 1 and 2.
//
// Sampler-match ("speculative-acceptance.md", "The rules", the default rule
// at T > 0) replaces pass 2 and the draw by:
//   2. match pass, one workgroup per (position, segment): the masses of p
//      below the drafted token t and in all, and sum p*q (the rule's
//      acceptance probability, "Verifying the gain").  The fresh draw from p
//      lands on t iff mass(< t) <= u*W < mass(< t) + p(t); the masses come from
//      float32 terms, so a decision closer to a boundary than they resolve is
//      taken again with float64 terms over the row;
//   3. the draw at the first mismatch (or the bonus row), as above from p.
#include "device.hpp"
#include "internal.hpp"

namespace vsel {

constexpr int PG = 4;  // 16-byte groups per lane per tile (float32 rows)

// Exclusive prefix sum over the workgroup (thread order), float64.
__device__ __forceinline__ double block_excl_scan_f64(SelShared& sh, double v, double* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    double o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) sh.ws[wave] = incl;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int q = 0; q < NWAVE; ++q) {
    if (q < wave) base += sh.ws[q];
    tot += sh.ws[q];
  }
  *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------- pass 2
// The accept test u * q(t) <= p(t) of one position in float64, from the row
// scan's log-sum-exps (kill_p / kill_q: the drafted token lies outside the
// filtered target / draft row).  Out of line, so that pass 2's position
// decision and the draws of the fused launch, which find the first rejection
// themselves, run the same code and take the same decision bit for bit.
__device__ __noinline__ uint32_t mrs_accept(float zt, float dt, double lp, double lq, float T, float u, bool kill_p,
                                            bool kill_q) {
  const double Td = T;
  double pt = exp((double)zt / Td - lp);
  double qt = exp((double)dt / Td - lq);
  if (kill_p) pt = 0.0;
  if (kill_q) qt = 0.0;
  return ((double)u * qt <= pt) ? 1u : 0u;
}

// (row, segment) of work item `l` of `n` items (a launch's items after its
// first ones), consecutive items on one XCD when n and the items before are
// whole multiples of the 8 XCDs (workgroups are dealt round-robin over them).
__device__ __forceinline__ Item work_item_at(uint32_t l, uint32_t n, bool xcd, int32_t S) {
  const uint32_t w = xcd ? (l & 7u) * (n >> 3) + (l >> 3) : l;
  const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(w / (uint32_t)S);
  return Item{row, (uint32_t)__builtin_amdgcn_readfirstlane(w - row * (uint32_t)S)};
}

// SP: also sum p*q per position (the sampler-match acceptance probability,
// reported beside sum min(p, q) as "Verifying the gain before trusting a
// throughput number" prints both closed forms), one more FMA per element.
// FUSED: the draws run in the same launch (coupling_draw_kernel) and own the
// emitted token at the first rejection L (or the bonus token).
template <bool VEC, bool FILT, bool SP, bool FUSED>
__device__ __forceinline__ void coupling_body(const SpecArgs& a, SelShared& sh, Item it) {
  constexpr int E = 4, TILE = NT * PG * E;
  const int tid = threadIdx.x;
  const int64_t pos = it.row;
  const int seg = (int)it.seg;
  const int64_t G = a.gamma;
  if (pos >= a.B * G) return;
  const int64_t b = pos / G, i = pos % G;
  const int64_t trow = b * (G + 1) + i, drow = b * G + i;
  const int64_t nT = a.B * (G + 1);
  const float* __restrict__ zr = a.tgt + trow * a.ld_t;
  const float* __restrict__ dr = a.dft + drow * a.ld_d;
  const bool bad = a.st_bad[trow] || a.st_bad[nT + drow];
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);

  // filtered rows: an element below its row's key floor has p (q) = 0
  const uint64_t kz = FILT ? a.kfl[trow] : 0ull, kd = FILT ? a.kfl[nT + drow] : 0ull;
  double tot = 0.0, tsp = 0.0;
  if (a.T > 0.0f && !bad) {
    // p = exp(z/T - lse_p) = exp2((z - m_z) c - (lse_p - m_z/T) log2e), the
    // exponent relative to the row maximum so that no float32 product carries
    // a large logit; the offset (at most log V) split in a float part and a
    // float factor
    const float c = a.lse_c;
    const float mz = a.st_max[trow], md = a.st_max[nT + drow];
    const double iT = 1.0 / (double)a.T, l2e = 1.4426950408889634;
    const double Lp = (a.st_lse[trow] - (double)mz * iT) * l2e, Lq = (a.st_lse[nT + drow] - (double)md * iT) * l2e;
    const float Lp_hi = (float)Lp, Lq_hi = (float)Lq;
    const float fp = (float)exp2(-(Lp - (double)Lp_hi)), fq = (float)exp2(-(Lq - (double)Lq_hi));
    // group j of this lane starts at element t0 + (j*NT + tid)*E
    auto pair = [&](const auto& gz, const auto& gd, int64_t t0) {
      constexpr int NGP = (int)(sizeof(gz) / sizeof(Group));
      float acc = 0.0f, acc2 = 0.0f;
#pragma unroll
      for (int j = 0; j < NGP; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float p = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gz[j].w[e]) - mz, c, -Lp_hi)) * fp;
          float q = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gd[j].w[e]) - md, c, -Lq_hi)) * fq;
          if constexpr (FILT) {
            const uint32_t x = (uint32_t)t0 + (uint32_t)((j * NT + tid) * E + e);
            if (comp_key(gz[j].w[e], x) < kz) p = 0.0f;
            if (comp_key(gd[j].w[e], x) < kd) q = 0.0f;
          }
          acc += fminf(p, q);
          if constexpr (SP) acc2 = fmaf(p, q, acc2);
        }
      tot += (double)acc;
      if constexpr (SP) tsp += (double)acc2;
    };
    const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
    const int64_t e_tiles = e_begin + (e_full - e_begin) / TILE * TILE;
    for (int64_t t0 = e_begin; t0 < e_tiles; t0 += TILE) {
      Group gz[PG], gd[PG];
      load_tile_full<float, PG, VEC>(gz, zr + t0);
      load_tile_full<float, PG, VEC>(gd, dr + t0);
      pair(gz, gd, t0);
    }
    if (e_tiles < e_full) {  // the last partial tile, its loads issued together
      Group gz[PG], gd[PG];
      load_tile<float, PG, VEC>(gz, zr, e_tiles, e_full);  // past e_full: -inf, so p = q = 0
      load_tile<float, PG, VEC>(gd, dr, e_tiles, e_full);
      pair(gz, gd, e_tiles);
    }
    if (tid == 0)
      for (int64_t x = e_full; x < e_end; ++x) {
        float p = __builtin_amdgcn_exp2f(fmaf(zr[x] - mz, c, -Lp_hi)) * fp;
        float q = __builtin_amdgcn_exp2f(fmaf(dr[x] - md, c, -Lq_hi)) * fq;
        if (FILT && comp_key(__float_as_uint(zr[x]), (uint32_t)x) < kz) p = 0.0f;
        if (FILT && comp_key(__float_as_uint(dr[x]), (uint32_t)x) < kd) q = 0.0f;
        tot += (double)fminf(p, q);
        if constexpr (SP) tsp += (double)(p * q);
      }
  }
  tot = block_sum_f64(sh, tot);
  if constexpr (SP) tsp = block_sum_f64(sh, tsp);
  if (a.S > 1) {
    if (tid == 0) {
      st_dev(&a.p_summin[pos * a.S + seg], tot);
      if constexpr (SP) st_dev(&a.p_wt[pos * a.S + seg], tsp);
    }
    if (!last_done(sh, a.tk_pos + pos, (uint32_t)a.S)) return;
    tot = merge_sum(sh, a.p_summin + pos * a.S, a.S);
    if constexpr (SP) tsp = merge_sum(sh, a.p_wt + pos * a.S, a.S);
  }
  // Position decision (one thread): coupling sum and the accept test.
  if (tid == 0) {
    const uint32_t t = a.tokens[pos];
    uint32_t flag;
    if (bad || t >= (uint64_t)a.V) {
      flag = 2u;  // the sequence fails closed
    } else if (a.T == 0.0f) {
      flag = (t == a.st_amax[trow]) ? 1u : 0u;
      tot = (a.st_amax[trow] == a.st_amax[nT + drow]) ? 1.0 : 0.0;
      tsp = tot;
    } else {
      const float zt = zr[t], dt = dr[t];
      flag = mrs_accept(zt, dt, a.st_lse[trow], a.st_lse[nT + drow], a.T, a.u_acc[pos],
                        FILT && comp_key(__float_as_uint(zt), t) < kz, FILT && comp_key(__float_as_uint(dt), t) < kd);
    }
    st_dev(&a.acc[pos], flag);
    if (a.summin) st_dev(&a.summin[pos], bad ? __builtin_nanf("") : (float)tot);
    if (SP) st_dev(&a.sumprod[pos], bad ? __builtin_nanf("") : (float)tsp);
  }
  if (!last_done(sh, a.tk_seq + b, (uint32_t)G)) return;
  if (tid < G) sh.hist[tid] = ld_dev(&a.acc[b * G + tid]);
  __syncthreads();
  if (tid != 0) return;

  // Sequence decision.  Fused with the draws, the token at the first
  // rejection (or the bonus token) is the draw's alone to write: this thread
  // leaves it, and a failed sequence has no draw.
  uint32_t* tm = a.tok_mrs + b * (G + 1);
  uint32_t* ta = a.tok_aa ? a.tok_aa + b * (G + 1) : nullptr;
  bool fail = a.st_bad[b * (G + 1) + G] != 0;
  for (int64_t q = 0; q < G; ++q) fail |= sh.hist[q] == 2u;
  int64_t L = G;
  for (int64_t q = 0; q < G; ++q)
    if (sh.hist[q] == 0u) {
      L = q;
      break;
    }
  for (int64_t q = 0; q <= G; ++q) {
    if (!FUSED || fail || q != L) tm[q] = kFail;
    if (ta) ta[q] = kFail;
  }
  if (fail) {
    a.len_mrs[b] = -1;
    if (a.len_aa) a.len_aa[b] = -1;
    if (a.summin)
      for (int64_t q = 0; q < G; ++q) st_dev(&a.summin[b * G + q], __builtin_nanf(""));
    if (SP)
      for (int64_t q = 0; q < G; ++q) st_dev(&a.sumprod[b * G + q], __builtin_nanf(""));
    a.draw_L[b] = -1;
    return;
  }
  int64_t Laa = G;
  for (int64_t q = 0; q < G; ++q)
    if (a.tokens[b * G + q] != a.st_amax[b * (G + 1) + q]) {
      Laa = q;
      break;
    }
  if (a.len_aa) a.len_aa[b] = (int32_t)Laa;
  if (ta) {
    for (int64_t q = 0; q < Laa; ++q) ta[q] = a.tokens[b * G + q];
    ta[Laa] = a.st_amax[b * (G + 1) + Laa];
  }
  if (a.T == 0.0f) {
    a.len_mrs[b] = (int32_t)Laa;
    for (int64_t q = 0; q < Laa; ++q) tm[q] = a.tokens[b * G + q];
    tm[Laa] = a.st_amax[b * (G + 1) + Laa];
    a.draw_L[b] = -1;
    return;
  }
  a.len_mrs[b] = (int32_t)L;
  for (int64_t q = 0; q < L; ++q) tm[q] = a.tokens[b * G + q];
  a.draw_L[b] = (int32_t)L;
}

template <bool VEC, bool FILT, bool SP>
__global__ __launch_bounds__(NT) void coupling_kernel(SpecArgs a) {
  __shared__ SelShared sh;
  coupling_body<VEC, FILT, SP, false>(a, sh, work_item(a.S));
}

// ---------------------------------------------------------------- sampler-match pass
// Float32 terms are within about 1e-6 of the total mass of their float64
// values on any row, so a decision farther than this from both boundaries of
// the drafted token's interval stands; a nearer one is taken again exactly.
constexpr double kMatchTol = 1e-5;

template <bool VEC, bool FILT>
__global__ __launch_bounds__(NT) void match_kernel(SpecArgs a) {
  constexpr int E = 4, TILE = NT * PG * E;
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t pos = it.row;
  const int seg = (int)it.seg;
  const int64_t G = a.gamma;
  if (pos >= a.B * G) return;
  const int64_t b = pos / G, i = pos % G;
  const int64_t trow = b * (G + 1) + i, drow = b * G + i;
  const int64_t nT = a.B * (G + 1);
  const float* __restrict__ zr = a.tgt + trow * a.ld_t;
  const float* __restrict__ dr = a.dft + drow * a.ld_d;
  const uint32_t t = a.tokens[pos];
  const bool bad = a.st_bad[trow] || a.st_bad[nT + drow] || t >= (uint64_t)a.V;
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);

  const uint64_t kz = FILT ? a.kfl[trow] : 0ull, kd = FILT ? a.kfl[nT + drow] : 0ull;
  double sp = 0.0, lo = 0.0, ws = 0.0;  // sum p q, mass of p below t, mass of p
  if (a.T > 0.0f && !bad) {
    // p = exp(z/T - lse_p) = exp2((z - m_z) c - (lse_p - m_z/T) log2e), the
    // exponent relative to the row maximum so that no float32 product carries
    // a large logit; the offset (at most log V) split in a float part and a
    // float factor
    const float c = a.lse_c;
    const float mz = a.st_max[trow], md = a.st_max[nT + drow];
    const double iT = 1.0 / (double)a.T, l2e = 1.4426950408889634;
    const double Lp = (a.st_lse[trow] - (double)mz * iT) * l2e, Lq = (a.st_lse[nT + drow] - (double)md * iT) * l2e;
    const float Lp_hi = (float)Lp, Lq_hi = (float)Lq;
    const float fp = (float)exp2(-(Lp - (double)Lp_hi)), fq = (float)exp2(-(Lq - (double)Lq_hi));
    // group j of this lane starts at element t0 + (j*NT + tid)*E
    auto pair = [&](const auto& gz, const auto& gd, int64_t t0) {
      constexpr int NGP = (int)(sizeof(gz) / sizeof(Group));
      float a_sp = 0.0f, a_lo = 0.0f, a_ws = 0.0f;
#pragma unroll
      for (int j = 0; j < NGP; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t x = (uint32_t)t0 + (uint32_t)((j * NT + tid) * E + e);
          float p = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gz[j].w[e]) - mz, c, -Lp_hi)) * fp;
          float q = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gd[j].w[e]) - md, c, -Lq_hi)) * fq;
          if constexpr (FILT) {
            if (comp_key(gz[j].w[e], x) < kz) p = 0.0f;
            if (comp_key(gd[j].w[e], x) < kd) q = 0.0f;
          }
          a_sp = fmaf(p, q, a_sp);
          a_ws += p;
          a_lo += x < t ? p : 0.0f;
        }
      sp += (double)a_sp;
      lo += (double)a_lo;
      ws += (double)a_ws;
    };
    const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
    const int64_t e_tiles = e_begin + (e_full - e_begin) / TILE * TILE;
    for (int64_t t0 = e_begin; t0 < e_tiles; t0 += TILE) {
      Group gz[PG], gd[PG];
      load_tile_full<float, PG, VEC>(gz, zr + t0);
      load_tile_full<float, PG, VEC>(gd, dr + t0);
      pair(gz, gd, t0);
    }
    if (e_tiles < e_full) {  // the last partial tile, its loads issued together
      Group gz[PG], gd[PG];
      load_tile<float, PG, VEC>(gz, zr, e_tiles, e_full);  // past e_full: -inf, so p = q = 0
      load_tile<float, PG, VEC>(gd, dr, e_tiles, e_full);
      pair(gz, gd, e_tiles);
    }
    if (tid == 0)
      for (int64_t x = e_full; x < e_end; ++x) {
        float p = __builtin_amdgcn_exp2f(fmaf(zr[x] - mz, c, -Lp_hi)) * fp;
        float q = __builtin_amdgcn_exp2f(fmaf(dr[x] - md, c, -Lq_hi)) * fq;
        if (FILT && comp_key(__float_as_uint(zr[x]), (uint32_t)x) < kz) p = 0.0f;
        if (FILT && comp_key(__float_as_uint(dr[x]), (uint32_t)x) < kd) q = 0.0f;
        sp += (double)(p * q);
        ws += (double)p;
        if ((uint64_t)x < t) lo += (double)p;
      }
  }
  sp = block_sum_f64(sh, sp);
  lo = block_sum_f64(sh, lo);
  ws = block_sum_f64(sh, ws);
  if (a.S > 1) {
    if (tid == 0) {
      st_dev(&a.p_summin[pos * a.S + seg], sp);
      st_dev(&a.p_low[pos * a.S + seg], lo);
      st_dev(&a.p_wt[pos * a.S + seg], ws);
    }
    if (!last_done(sh, a.tk_pos + pos, (uint32_t)a.S)) return;
    sp = merge_sum(sh, a.p_summin + pos * a.S, a.S);
    lo = merge_sum(sh, a.p_low + pos * a.S, a.S);
    ws = merge_sum(sh, a.p_wt + pos * a.S, a.S);
  }
  // Position decision (every thread holds the same sums, so the branches
  // below are uniform): 1 the fresh draw is t, 0 it is not, 2 fail closed.
  uint32_t flag;
  if (bad) {
    flag = 2u;
  } else if (a.T == 0.0f) {
    flag = (t == a.st_amax[trow]) ? 1u : 0u;
    sp = (a.st_amax[trow] == a.st_amax[nT + drow]) ? 1.0 : 0.0;
  } else {
    const double Td = a.T, lse = a.st_lse[trow];
    const double pt = (FILT && comp_key(__float_as_uint(zr[t]), t) < kz) ? 0.0 : exp((double)zr[t] / Td - lse);
    const double u = (double)a.u_match[b * (G + 1) + i];
    const double target = u * ws, tol = kMatchTol * ws;
    if (target >= lo + tol && target < lo + pt - tol) {
      flag = 1u;
    } else if (target < lo - tol || target >= lo + pt + tol) {
      flag = 0u;
    } else {
      // too close to call: the masses again, from float64 terms
      double l2 = 0.0, w2 = 0.0;
      for (int64_t x = tid; x < a.V; x += NT) {
        const double px =
            (FILT && comp_key(__float_as_uint(zr[x]), (uint32_t)x) < kz) ? 0.0 : exp((double)zr[x] / Td - lse);
        w2 += px;
        if ((uint64_t)x < t) l2 += px;
      }
      l2 = block_sum_f64(sh, l2);
      w2 = block_sum_f64(sh, w2);
      const double tg = u * w2;
      flag = (l2 <= tg && tg < l2 + pt) ? 1u : 0u;
    }
  }
  if (tid == 0) {
    st_dev(&a.acc[pos], flag);
    if (a.sumprod) st_dev(&a.sumprod[pos], bad ? __builtin_nanf("") : (float)sp);
  }
  if (!last_done(sh, a.tk_seq + b, (uint32_t)G)) return;
  if (tid < G) sh.hist[tid] = ld_dev(&a.acc[b * G + tid]);
  __syncthreads();
  if (tid != 0) return;

  // Sequence decision: the chain runs to the first position whose draw is
  // not the drafted token (gamma: the bonus row); the draw there is emitted.
  uint32_t* tk = a.tok_sm + b * (G + 1);
  bool fail = a.st_bad[b * (G + 1) + G] != 0;
  for (int64_t q = 0; q < G; ++q) fail |= sh.hist[q] == 2u;
  for (int64_t q = 0; q <= G; ++q) tk[q] = kFail;
  if (fail) {
    a.len_sm[b] = -1;
    if (a.sumprod)
      for (int64_t q = 0; q < G; ++q) st_dev(&a.sumprod[b * G + q], __builtin_nanf(""));
    a.draw_L[b] = -1;
    return;
  }
  int64_t L = G;
  for (int64_t q = 0; q < G; ++q)
    if (sh.hist[q] == 0u) {
      L = q;
      break;
    }
  a.len_sm[b] = (int32_t)L;
  for (int64_t q = 0; q < L; ++q) tk[q] = a.tokens[b * G + q];
  if (a.T == 0.0f) {  // the sampler is argmax: its draw is the argmax
    tk[L] = a.st_amax[b * (G + 1) + L];
    a.draw_L[b] = -1;
    return;
  }
  a.draw_L[b] = (int32_t)L;
}

// ---------------------------------------------------------------- pass 3
// ---------------------------------------------------------------- pass 4 (and the full-row draw)
// An inverse-CDF draw in id order over W = sum of weights, in three levels:
// segment masses, 256-element chunk masses, then one element per thread.
// Every mass is a float64 sum; a segment's mass is the in-order sum of its
// chunk masses, so the levels agree up to the last bits of the final scan.

// Source of a draw: weight w(x) >= 0 of row element x.
//   residual: max(p - q, 0), p = exp(z/T - lp), q = exp(d/T - lq)
//   plain:    exp((z - m) / T), proportional to p (u*W does not see the scale)
//   (plain only) elements below thr weigh nothing: the sampler chain's
//   threshold filters over a whole row
//   filtered p and q: an element whose composite key is below kz (of the
//   target row) or kd (of the draft row) has p = 0 or q = 0
template <typename DT>
struct DrawSrc {
  const DT* z;
  const float* d;  // null: plain
  double lp, lq, m, T;
  int64_t V;
  double thr = -__builtin_inf();
  uint64_t kz = 0, kd = 0;
  double iT = 1.0;              // 1 / T
  const double* e2 = nullptr;   // the exp table in LDS (init_e2)
  bool vz = false, vd = false;  // the rows start and stride on 16 bytes
  __device__ __forceinline__ float zv(int64_t x) const { return __uint_as_float(gbits_at<DT>(z, x)); }
  // (every exponent is at most 0 up to rounding: lp and lq are log-sum-exps
  // of the rows at T, m their maxima)
  __device__ __forceinline__ double w(float zx, float dx, int64_t x) const {
    const bool pk = kz == 0 || comp_key(__float_as_uint(zx), (uint32_t)x) >= kz;
    if (d) {
      const bool qk = kd == 0 || comp_key(__float_as_uint(dx), (uint32_t)x) >= kd;
      const double p = pk ? exp_le0((double)zx * iT - lp, e2) : 0.0;
      const double q = qk ? exp_le0((double)dx * iT - lq, e2) : 0.0;
      return p > q ? p - q : 0.0;
    }
    return pk && (double)zx >= thr ? exp_le0(((double)zx - m) * iT, e2) : 0.0;
  }
};

// Elements x .. x+3 of a row as float32 (fill at and past lim): one 16-byte
// (float32) or 8-byte (bfloat16) load when the row is aligned and all four are
// in range, else element loads (at `safe`, a valid index, for those past lim).
struct F4 {
  float v[4];
};
template <typename DT>
__device__ __forceinline__ F4 row4(const DT* __restrict__ row, int64_t x, int64_t lim, bool vec, float fill,
                                   int64_t safe) {
  F4 o;
  if (vec && x + 3 < lim) {
    if constexpr (sizeof(DT) == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + x);
#pragma unroll
      for (int e = 0; e < 4; ++e) o.v[e] = __uint_as_float(v[e]);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(row + x);
      o.v[0] = __uint_as_float(v.x << 16);
      o.v[1] = __uint_as_float(v.x & 0xFFFF0000u);
      o.v[2] = __uint_as_float(v.y << 16);
      o.v[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = x + e < lim;
      const float v = __uint_as_float(gbits_at<DT>(row, in ? x + e : safe));
      o.v[e] = in ? v : fill;
    }
  }
  return o;
}

// Chunk masses of segment [e_begin, e_end): each wave takes CW chunks per
// step (4 CW loads per lane in flight), reduces each chunk's 256 weights (4
// per lane) in float64, and writes the masses to `cm` (LDS) and `pc` (global,
// indexed from the segment's first chunk).  Returns the segment mass in
// thread 0: the in-order sum of its chunk masses.  (CW = 2 in the launch that
// shares its workgroups' registers with pass 2, 4 in launches of their own.)
template <int CW, class Src>
__device__ double chunk_masses(const Src& r, int64_t e_begin, int64_t e_end, double* cm, double* pc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (int)((e_end - e_begin + kChunk - 1) / kChunk);
  for (int q0 = 0; q0 < nch; q0 += NWAVE * CW) {
    float zz[CW][4], dd[CW][4];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int q = q0 + wave * CW + j;
      const int64_t x0 = e_begin + (int64_t)q * kChunk + lane * 4;
      const int64_t lim = q < nch ? e_end : x0;  // past the segment: weight 0
      const F4 fz = row4(r.z, x0, lim, r.vz, -__builtin_inff(), e_begin);
      const F4 fd = r.d ? row4(r.d, x0, lim, r.vd, 0.0f, e_begin) : F4{{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zz[j][e] = fz.v[e];
        dd[j][e] = fd.v[e];
      }
    }
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int q = q0 + wave * CW + j;
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) s += r.w(zz[j][e], dd[j][e], e_begin + (int64_t)q * kChunk + lane * 4 + e);
      s = wave_sum_f64(s);
      if (lane == 0 && q < nch) {
        cm[q] = s;
        st_dev(&pc[q], s);
      }
    }
  }
  __syncthreads();
  double tot = 0.0;
  if (tid == 0)
    for (int q = 0; q < nch; ++q) tot += cm[q];
  return tot;
}

// The first of n masses v[0..n) (LDS) whose running sum passes t (t <
// cum + v[i]), by wave 0: each lane sums a run of ceil(n / 64) consecutive
// masses in order, the runs are prefixed across the lanes (float64, a fixed
// order), and the lane holding the crossing walks its run.  Returns the
// index in every lane of wave 0 and sets *rem to the part of t past the
// masses before it; with no crossing (rounding at the very top) the last
// positive mass (index 0 if none), *rem its mass.  total: the sum of the
// runs, for callers that need W before choosing t (then t = scale * W).
__device__ __forceinline__ int wave_pick_mass(const double* v, int n, double scale, bool scale_by_total, double t,
                                              double* rem, double* total) {
  const int lane = threadIdx.x & 63;
  const int R = (n + 63) / 64;
  const int lo = min(n, lane * R), hi = min(n, lo + R);
  double run = 0.0;
  for (int i = lo; i < hi; ++i) run += v[i];
  double incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const double W = __shfl(incl, 63);
  if (scale_by_total) t = scale * W;
  double c = __shfl_up(incl, 1);
  if (lane == 0) c = 0.0;
  int found = -1, lastpos = -1;
  double r = 0.0;
  for (int i = lo; i < hi; ++i) {
    if (found < 0 && t < c + v[i]) {
      found = i;
      r = t - c;
    }
    if (v[i] > 0.0) lastpos = i;
    c += v[i];
  }
  const uint64_t hit = __ballot(found >= 0);
  int pick;
  double rr;
  if (hit) {
    const int l = __builtin_ctzll(hit);
    pick = __shfl(found, l);
    rr = __shfl(r, l);
  } else {
    const uint64_t pos = __ballot(lastpos >= 0);
    const int l = pos ? 63 - __builtin_clzll(pos) : 0;
    pick = pos ? __shfl(lastpos, l) : 0;
    rr = v[pick];
  }
  *rem = rr;
  *total = W;
  return pick;
}

// Whether any of v[0..n) (LDS, n <= 4 * 64) is positive, by wave 0 (a sum of
// such nonnegative masses is positive exactly then).
__device__ __forceinline__ bool wave_any_positive(const double* v, int n) {
  const int lane = threadIdx.x & 63;
  bool any = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) any = any || (q * 64 + lane < n && v[q * 64 + lane] > 0.0);
  return __ballot(any) != 0ull;
}

// The draw itself (one workgroup): segment, then chunk, then element.  pw
// (LDS) holds the S segment masses, pc (global) the row's chunk masses; cm is
// LDS room for kChunksPerSeg chunk masses.
// Returns the token in every thread; *W_out (thread 0) is the total mass.
template <class Src>
__device__ uint32_t draw_pick(SelShared& sh, const Src& r, const double* pw, const double* pc, int S,
                              int64_t seg_len, double u, double* W_out, double* cm) {
  const int tid = threadIdx.x;
  __shared__ int s_seg, s_ch;
  __shared__ double s_in;
  __shared__ uint32_t s_tok;
  if (tid < 64) {
    double rem, W;
    const int pick = wave_pick_mass(pw, S, u, true, 0.0, &rem, &W);
    if (tid == 0) {
      s_seg = pick;
      s_in = rem;
      s_tok = kFail;
      *W_out = W;
    }
  }
  __syncthreads();
  const int64_t e_begin = (int64_t)s_seg * seg_len, e_end = min(r.V, e_begin + seg_len);
  const int nch = (int)((e_end - e_begin + kChunk - 1) / kChunk);
  for (int q = tid; q < nch; q += NT) cm[q] = ld_dev(&pc[e_begin / kChunk + q]);
  __syncthreads();
  if (tid < 64) {
    double rem, unused;
    const int pick = wave_pick_mass(cm, nch, 0.0, false, s_in, &rem, &unused);
    if (tid == 0) {
      s_ch = pick;
      s_in = rem;
    }
  }
  __syncthreads();
  const int64_t c0 = e_begin + (int64_t)s_ch * kChunk;
  const int64_t x = c0 + tid;
  const double wx = x < e_end ? r.w(r.zv(x), r.d ? r.d[x] : 0.0f, x) : 0.0;
  double total;
  const double excl = block_excl_scan_f64(sh, wx, &total);
  const double t2 = s_in;
  if (excl <= t2 && t2 < excl + wx) s_tok = (uint32_t)x;
  __syncthreads();
  if (tid == 0 && s_tok == kFail) {  // rounding: the chunk's last element with weight
    for (int64_t y = min(e_end, c0 + kChunk) - 1; y >= c0; --y)
      if (r.w(r.zv(y), r.d ? r.d[y] : 0.0f, y) > 0.0) {
        s_tok = (uint32_t)y;
        break;
      }
    if (s_tok == kFail) s_tok = (uint32_t)c0;
  }
  __syncthreads();
  return s_tok;
}

// The residual draw of modified rejection sampling in one pass.  With
// P = exp((z - m_z)/T) and Q = exp((d - m_d)/T) (m the rows' maxima) and
// Sp, Sq their float64 row sums, p = P/Sp and q = Q/Sq, so
//   max(p - q, 0) = P/Sp - Q/Sq   where D = (z - m_z)/T - (d - m_d)/T > log(Sp/Sq),
// and 0 elsewhere.  The pass sums Sp and Sq and, per 256-element chunk, P and
// Q over the elements with D above the threshold the row scan's log-sum-exps
// give (they approximate the rows' sums to within about the rows' entropy in
// bits times 2^-24, well inside kBand); a chunk holding an element within kBand of it is flagged, and
// the last workgroup recomputes it element by element once Sp and Sq are
// exact.  Every other chunk's residual mass is then A/Sp - B/Sq.
constexpr double kBand = 1e-5;

struct ResidSrc {
  const float* z;
  const float* d;
  double mz, md, iT, iSp, iSq;
  int64_t V;
  const double* e2;
  bool vz, vd;  // the rows start and stride on 16 bytes
  __device__ __forceinline__ float zv(int64_t x) const { return z[x]; }
  __device__ __forceinline__ double w(float zx, float dx, int64_t) const {
    const double p = exp_le0(((double)zx - mz) * iT, e2) * iSp, q = exp_le0(((double)dx - md) * iT, e2) * iSq;
    return p > q ? p - q : 0.0;
  }
};

// Chunk sums of segment [e_begin, e_end) for the residual draw (chunks
// indexed from the segment's first in pa, pb, pf); returns (every thread) the
// segment's sums of P and Q.
__device__ void resid_chunks(SelShared& sh, const ResidSrc& r, double theta, int64_t e_begin, int64_t e_end,
                             double* pa, double* pb, uint32_t* pf, double* sp_out, double* sq_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int CW = 2;  // chunks per wave per step (the registers of pass 2's workgroups bound it)
  const int nch = (int)((e_end - e_begin + kChunk - 1) / kChunk);
  double sp = 0.0, sq = 0.0;
  for (int q0 = 0; q0 < nch; q0 += NWAVE * CW) {
    float zz[CW][4], dd[CW][4];
#pragma unroll
    for (int j = 0; j < CW; ++j) {  // past the segment: P = Q = 0, on neither side
      const int q = q0 + wave * CW + j;
      const int64_t x0 = e_begin + (int64_t)q * kChunk + lane * 4;
      const int64_t lim = q < nch ? e_end : x0;
      const F4 fz = row4(r.z, x0, lim, r.vz, -__builtin_inff(), e_begin);
      const F4 fd = row4(r.d, x0, lim, r.vd, -__builtin_inff(), e_begin);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zz[j][e] = fz.v[e];
        dd[j][e] = fd.v[e];
      }
    }
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int q = q0 + wave * CW + j;
      double A = 0.0, B = 0.0;
      bool near = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double az = ((double)zz[j][e] - r.mz) * r.iT, ad = ((double)dd[j][e] - r.md) * r.iT;
        const double P = exp_le0(az, r.e2), Q = exp_le0(ad, r.e2);
        sp += P;
        sq += Q;
        const double D = az - ad;  // NaN (both masked) counts on neither side
        if (D > theta + kBand) {
          A += P;
          B += Q;
        } else if (D >= theta - kBand) {
          near = true;
        }
      }
      A = wave_sum_f64(A);
      B = wave_sum_f64(B);
      const bool flag = __ballot(near) != 0ull;
      if (lane == 0 && q < nch) {
        st_dev(&pa[q], A);
        st_dev(&pb[q], B);
        st_dev(&pf[q], flag ? 1u : 0u);
      }
    }
  }
  *sp_out = block_sum_f64(sh, sp);
  *sq_out = block_sum_f64(sh, sq);
}

// The residual draw of sequence b at its first rejection L (unfiltered p and
// q), one workgroup per segment of the row pair; the last one draws.
__device__ void resid_draw(const SpecArgs& a, SelShared& sh, int64_t b, int seg, int32_t L, const double* e2,
                           double* cmw) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t G = a.gamma, nT = a.B * (G + 1);
  const int64_t trow = b * (G + 1) + L, drow = nT + b * G + L;
  ResidSrc r;
  r.z = a.tgt + trow * a.ld_t;
  r.d = a.dft + (b * G + L) * a.ld_d;
  r.mz = a.st_max[trow];
  r.md = a.st_max[drow];
  r.iT = 1.0 / (double)a.T;
  r.iSp = r.iSq = 1.0;
  r.V = a.V;
  r.e2 = e2;
  r.vz = a.vec_t != 0;
  r.vd = a.vec_d != 0;
  // log(Sp/Sq), approximately, from the row scan's log-sum-exps at T
  const double theta = (a.st_lse[trow] - r.mz * r.iT) - (a.st_lse[drow] - r.md * r.iT);
  double* pa = a.p_c + b * a.nchunk;
  double* pb = a.p_cb + b * a.nchunk;
  uint32_t* pf = a.p_cf + b * a.nchunk;
  const int64_t e_begin = (int64_t)seg * a.dseg, e_end = min(a.V, e_begin + a.dseg), c0 = e_begin / kChunk;
  double sp, sq;
  resid_chunks(sh, r, theta, e_begin, e_end, pa + c0, pb + c0, pf + c0, &sp, &sq);
  double* ps = a.p_lse + b * 2 * a.dS;  // the segments' Sp, then their Sq
  if (tid == 0) {
    st_dev(&ps[seg], sp);
    st_dev(&ps[a.dS + seg], sq);
  }
  if (!last_done(sh, a.tk_draw + b, (uint32_t)a.dS)) return;
  // ---- the row's last workgroup
  const double Sp = merge_sum(sh, ps, a.dS), Sq = merge_sum(sh, ps + a.dS, a.dS);
  r.iSp = 1.0 / Sp;
  r.iSq = 1.0 / Sq;
  // each chunk's residual mass: A/Sp - B/Sq, or element by element where
  // flagged; rows of up to kRcLds chunks also keep them in LDS, so that the
  // segment sums below read LDS instead of global memory
  constexpr int kRcPer = 4, kRcLds = kRcPer * NT;
  static_assert(kRcLds <= kChunksPerSeg, "the chunk masses live in the kernel's chunk buffer");
  double* rc = cmw;
  __shared__ uint16_t s_list[kRcLds];
  __shared__ uint32_t s_n;
  const int64_t nch = a.nchunk;
  const bool in_lds = nch <= kRcLds;
  for (int64_t cb = 0; cb < nch; cb += kRcLds) {
    if (tid == 0) s_n = 0u;
    double A[kRcPer], B[kRcPer];
    uint32_t F[kRcPer];
#pragma unroll
    for (int q = 0; q < kRcPer; ++q) {  // every load issued before any is used
      const int64_t c = cb + q * NT + tid;
      A[q] = c < nch ? ld_dev(&pa[c]) : 0.0;
      B[q] = c < nch ? ld_dev(&pb[c]) : 0.0;
      F[q] = c < nch ? ld_dev(&pf[c]) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kRcPer; ++q) {
      const int64_t c = cb + q * NT + tid;
      if (c >= nch) continue;
      if (F[q]) {
        s_list[atomicAdd(&s_n, 1u)] = (uint16_t)(c - cb);
      } else {
        const double m = fmax(A[q] * r.iSp - B[q] * r.iSq, 0.0);
        st_dev(&pa[c], m);
        if (in_lds) rc[c] = m;
      }
    }
    __syncthreads();
    const uint32_t n = s_n;
    for (uint32_t k = (uint32_t)wave; k < n; k += NWAVE) {
      const int64_t cc = cb + s_list[k];
      double m = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t x = cc * kChunk + lane * 4 + e;
        if (x < a.V) m += r.w(r.z[x], r.d[x], x);
      }
      m = wave_sum_f64(m);
      if (lane == 0) {
        st_dev(&pa[cc], m);
        if (in_lds) rc[cc] = m;
      }
    }
    __syncthreads();
  }
  // segment masses: the in-order sums of their chunk masses
  __shared__ double pw[kMaxSegments];
  __shared__ int s_degen;
  if (tid < a.dS) {
    const int64_t per = a.dseg / kChunk, c_lo = (int64_t)tid * per, c_hi = min(nch, c_lo + per);
    double t = 0.0;
    if (in_lds)
      for (int64_t c = c_lo; c < c_hi; ++c) t += rc[c];
    else
      for (int64_t c = c_lo; c < c_hi; ++c) t += ld_dev(&pa[c]);
    pw[tid] = t;
  }
  __syncthreads();
  if (tid < 64) {
    const bool pos = wave_any_positive(pw, a.dS);
    if (tid == 0) s_degen = pos ? 0 : 1;
  }
  __syncthreads();
  double W;
  uint32_t tok;
  if (!s_degen) {
    tok = draw_pick(sh, r, pw, pa, a.dS, a.dseg, (double)a.u_res[b * G + L], &W, cmw);
  } else {  // the residual sums to 0 (p <= q everywhere): draw from p
    DrawSrc<float> r2;
    r2.z = r.z;
    r2.d = nullptr;
    r2.lp = r2.lq = 0.0;
    r2.m = r.mz;
    r2.T = a.T;
    r2.iT = r.iT;
    r2.e2 = e2;
    r2.V = a.V;
    r2.vz = r.vz;
    for (int sg = 0; sg < a.dS; ++sg) {
      const int64_t eb = (int64_t)sg * a.dseg, ee = min(a.V, eb + a.dseg);
      const double m2 = chunk_masses<2>(r2, eb, ee, cmw, pa + eb / kChunk);
      if (tid == 0) pw[sg] = m2;
      __syncthreads();
    }
    tok = draw_pick(sh, r2, pw, pa, a.dS, a.dseg, (double)a.u_res[b * G + L], &W, cmw);
  }
  if (tid == 0) a.tok_mrs[b * (G + 1) + L] = tok;
}

// One workgroup's share of sequence b's draw at L (L < gamma: the residual
// at the first rejection, or the sampler-match draw at the first mismatch;
// L = gamma: the bonus token), segment seg of the draw row.  FUSED: the draws
// of unfiltered modified rejection sampling in pass 2's launch.
template <bool FUSED>
__device__ __forceinline__ void draw_item(const SpecArgs& a, SelShared& sh, int64_t b, int seg, int32_t L) {
  constexpr int CW = FUSED ? 2 : 4;
  __shared__ double cmw[kChunksPerSeg];
  const int tid = threadIdx.x;
  const int64_t G = a.gamma;
  __shared__ double e2[64];
  init_e2(e2);
  if (FUSED && L < G && !a.kfl) {  // the residual draw of unfiltered p and q
    resid_draw(a, sh, b, seg, L, e2, cmw);
    return;
  }
  DrawSrc<float> r;
  r.T = a.T;
  r.iT = 1.0 / r.T;
  r.e2 = e2;
  r.V = a.V;
  r.vz = a.vec_t != 0;
  r.vd = a.vec_d != 0;
  double u;
  const int64_t nT = a.B * (G + 1);
  if (a.match) {  // sampler-match: a fresh draw from p at row L
    r.z = a.tgt + (b * (G + 1) + L) * a.ld_t;
    r.d = nullptr;
    r.lp = r.lq = 0.0;
    r.m = a.st_max[b * (G + 1) + L];
    u = a.u_match[b * (G + 1) + L];
  } else if (L < G) {
    r.z = a.tgt + (b * (G + 1) + L) * a.ld_t;
    r.d = a.dft + (b * G + L) * a.ld_d;
    // filtered: the exact kept-set lse of the filter pass
    r.lp = a.st_lse[b * (G + 1) + L];
    r.lq = a.st_lse[nT + b * G + L];
    r.m = 0.0;
    u = a.u_res[b * G + L];
  } else {
    r.z = a.tgt + (b * (G + 1) + G) * a.ld_t;
    r.d = nullptr;
    r.lp = r.lq = 0.0;
    r.m = a.st_max[b * (G + 1) + G];
    u = a.u_bon[b];
  }
  if (a.kfl) {
    r.kz = a.kfl[b * (G + 1) + (a.match ? L : min((int64_t)L, G))];
    r.kd = L < G ? a.kfl[nT + b * G + L] : 0ull;
  }
  double* pc = a.p_c + b * a.nchunk;
  const int64_t e_begin = (int64_t)seg * a.dseg, e_end = min(a.V, e_begin + a.dseg);
  const double ms = chunk_masses<CW>(r, e_begin, e_end, cmw, pc + e_begin / kChunk);
  if (tid == 0) st_dev(&a.p_w[b * a.dS + seg], ms);
  if (!last_done(sh, a.tk_draw + b, (uint32_t)a.dS)) return;
  __shared__ double pw[kMaxSegments];
  if (tid < a.dS) pw[tid] = ld_dev(&a.p_w[b * a.dS + tid]);
  __syncthreads();
  // Degenerate residual (p <= q everywhere): draw from p instead.
  __shared__ int s_degen;
  if (tid < 64) {
    const bool degen = r.d != nullptr && !wave_any_positive(pw, a.dS);
    if (tid == 0) s_degen = degen ? 1 : 0;
  }
  __syncthreads();
  if (s_degen) {
    r.d = nullptr;
    r.m = a.st_max[b * (G + 1) + L];
    for (int sg = 0; sg < a.dS; ++sg) {
      const int64_t eb = (int64_t)sg * a.dseg, ee = min(a.V, eb + a.dseg);
      const double m2 = chunk_masses<CW>(r, eb, ee, cmw, pc + eb / kChunk);
      if (tid == 0) pw[sg] = m2;
      __syncthreads();
    }
  }
  double W;
  const uint32_t tok = draw_pick(sh, r, pw, pc, a.dS, a.dseg, u, &W, cmw);
  if (tid == 0) (a.match ? a.tok_sm : a.tok_mrs)[b * (G + 1) + L] = tok;
}

// The draw as a launch of its own, after pass 2 has decided L: sampler-match,
// whose first mismatch needs pass 2's masses (modified rejection sampling
// draws in pass 2's launch).
__global__ __launch_bounds__(NT) void spec_draw_kernel(SpecArgs a) {
  __shared__ SelShared sh;
  const Item it = work_item(a.dS);
  const int64_t b = it.row;
  if (b >= a.B) return;
  const int32_t L = a.draw_L[b];
  if (L < 0) return;
  draw_item<false>(a, sh, b, (int)it.seg, L);
}

// First rejection of sequence b under modified rejection sampling (gamma:
// every draft accepted), or -1 where the sequence fails closed: pass 2's
// position and sequence decisions, taken again from the row scan's results
// (and the filter pass's, FILT) with the same accept function (T > 0).
template <bool FILT>
__device__ __forceinline__ int32_t first_reject(const SpecArgs& a, SelShared& sh, int64_t b) {
  const int tid = threadIdx.x;
  const int64_t G = a.gamma, nT = a.B * (G + 1);
  __shared__ int32_t s_L;
  if (tid < G) {
    const int64_t pos = b * G + tid, trow = b * (G + 1) + tid, drow = b * G + tid;
    const uint32_t t = a.tokens[pos];
    uint32_t flag = 2u;
    if (!a.st_bad[trow] && !a.st_bad[nT + drow] && t < (uint64_t)a.V) {
      const float zt = a.tgt[trow * a.ld_t + t], dt = a.dft[drow * a.ld_d + t];
      const bool kill_p = FILT && comp_key(__float_as_uint(zt), t) < a.kfl[trow];
      const bool kill_q = FILT && comp_key(__float_as_uint(dt), t) < a.kfl[nT + drow];
      flag = mrs_accept(zt, dt, a.st_lse[trow], a.st_lse[nT + drow], a.T, a.u_acc[pos], kill_p, kill_q);
    }
    sh.hist[tid] = flag;
  }
  __syncthreads();
  if (tid == 0) {
    bool fail = a.st_bad[b * (G + 1) + G] != 0;
    int32_t L = (int32_t)G;
    for (int64_t q = 0; q < G; ++q) fail |= sh.hist[q] == 2u;
    for (int64_t q = 0; q < G; ++q)
      if (sh.hist[q] == 0u) {
        L = (int32_t)q;
        break;
      }
    s_L = fail ? -1 : L;
  }
  __syncthreads();
  return s_L;
}

// Pass 2 and the draws of modified rejection sampling (T > 0) in one launch.
// The first B * dS workgroups are the draws (dispatched first, so that their
// float64 work overlaps the coupling pass's stream); each finds its
// sequence's first rejection itself, so it need not wait for pass 2.  The
// rest are pass 2's (position, segment) items.
template <bool VEC, bool FILT, bool SP>
__global__ __launch_bounds__(NT) void coupling_draw_kernel(SpecArgs a) {
  __shared__ SelShared sh;
  const uint32_t nd = (uint32_t)(a.B * a.dS);
  if (blockIdx.x < nd) {
    const uint32_t b = blockIdx.x / (uint32_t)a.dS;
    const int32_t L = first_reject<FILT>(a, sh, b);
    if (L >= 0) draw_item<true>(a, sh, b, (int)(blockIdx.x - b * (uint32_t)a.dS), L);
    return;
  }
  const uint32_t n = gridDim.x - nd;
  coupling_body<VEC, FILT, SP, true>(a, sh, work_item_at(blockIdx.x - nd, n, (nd & 7u) == 0 && (n & 7u) == 0, a.S));
}

template <typename DT>
__global__ __launch_bounds__(NT) void row_draw_kernel(DrawArgs a) {
  __shared__ SelShared sh;
  __shared__ double cmw[kChunksPerSeg];
  const int tid = threadIdx.x;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  if (a.st_bad[row]) {
    if (seg == 0 && tid == 0) {
      a.out_token[row] = kFail;
      if (a.out_logp) a.out_logp[row] = __builtin_nanf("");
    }
    return;
  }
  __shared__ double e2[64];
  init_e2(e2);
  DrawSrc<DT> r;
  r.z = reinterpret_cast<const DT*>(a.x) + row * a.ld;
  r.d = nullptr;
  r.lp = r.lq = 0.0;
  r.m = a.st_max[row];
  r.T = a.T;
  r.iT = 1.0 / r.T;
  r.e2 = e2;
  r.V = a.V;
  r.vz = a.vec != 0;
  if (a.top_n_sigma > 0.0f) r.thr = r.m - (double)a.top_n_sigma * a.sigma[row];
  if (a.min_p > 0.0f) r.thr = fmax(r.thr, r.m + log((double)a.min_p));
  double* pc = a.p_c + row * a.nchunk;
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);
  const double ms = chunk_masses<4>(r, e_begin, e_end, cmw, pc + e_begin / kChunk);
  if (tid == 0) st_dev(&a.p_w[row * a.S + seg], ms);
  if (!last_done(sh, a.tickets + row, (uint32_t)a.S)) return;
  __shared__ double pw[kMaxSegments];
  if (tid < a.S) pw[tid] = ld_dev(&a.p_w[row * a.S + tid]);
  __syncthreads();
  double W;
  const uint32_t tok = draw_pick(sh, r, pw, pc, a.S, a.seg_len, (double)a.u[row], &W, cmw);
  if (tid == 0) {
    a.out_token[row] = tok;
    if (a.out_logp) a.out_logp[row] = (float)(((double)r.zv(tok) - r.m) / r.T - log(W));
  }
}

// Pass 2: at T > 0 with the draws in the same launch (their workgroups
// first), at T = 0 (no draw) alone.
template <bool VEC, bool FILT>
static void launch_coupling(bool sp, const SpecArgs& a, hipStream_t s) {
  const unsigned npos = (unsigned)(a.B * a.gamma * a.S);
  if (a.T > 0.0f) {
    const dim3 grid((unsigned)(a.B * a.dS) + npos);
    if (sp)
      hipLaunchKernelGGL((coupling_draw_kernel<VEC, FILT, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((coupling_draw_kernel<VEC, FILT, false>), grid, dim3(NT), 0, s, a);
  } else if (sp) {
    hipLaunchKernelGGL((coupling_kernel<VEC, FILT, true>), dim3(npos), dim3(NT), 0, s, a);
  } else {
    hipLaunchKernelGGL((coupling_kernel<VEC, FILT, false>), dim3(npos), dim3(NT), 0, s, a);
  }
}

hipError_t launch_spec(const SpecArgs& a, hipStream_t s) {
  const bool vec = a.vec_t && a.vec_d;
  const bool sp = a.sumprod != nullptr;
  if (a.kfl) {
    if (vec)
      launch_coupling<true, true>(sp, a, s);
    else
      launch_coupling<false, true>(sp, a, s);
  } else {
    if (vec)
      launch_coupling<true, false>(sp, a, s);
    else
      launch_coupling<false, false>(sp, a, s);
  }
  return hipGetLastError();
}

hipError_t launch_spec_match(const SpecArgs& a, hipStream_t s) {
  const unsigned npos = (unsigned)(a.B * a.gamma * a.S);
  const bool vec = a.vec_t && a.vec_d;
  if (a.kfl) {
    if (vec)
      hipLaunchKernelGGL((match_kernel<true, true>), dim3(npos), dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((match_kernel<false, true>), dim3(npos), dim3(NT), 0, s, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((match_kernel<true, false>), dim3(npos), dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((match_kernel<false, false>), dim3(npos), dim3(NT), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.T == 0.0f) return e;
  hipLaunchKernelGGL(spec_draw_kernel, dim3((unsigned)(a.B * a.dS)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_draw_rows(int dtype, const DrawArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.S));
  if (dtype == 0)
    hipLaunchKernelGGL(row_draw_kernel<float>, grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(row_draw_kernel<uint16_t>, grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace vsel
