// spec.hip -- speculative-decoding acceptance on the device, and the
// full-row categorical draw.
//
// Modified rejection sampling ("speculative-acceptance.md", "Modified
// rejection sampling"; the exact CPU acceptance of "Chapter 21", section
// 21.9) needs, per verified position, two full-vocabulary reductions (the
// pages' MLX version pays them as extra passes plus a host sync per
// position).  Here the whole batch runs in four launches on one stream and
// nothing returns to the host:
//   1. row scan (scan.hip) over all target and draft rows: argmax, maximum,
//      latch, log-sum-exp at T;
//   2. coupling pass, one workgroup per (position, segment): p = exp(z/T -
//      lse_p), q = exp(d/T - lse_q), sum of min(p, q) (the acceptance ceiling
//      of "The acceptance ceiling").  The last workgroup of a position decides
//      u * q(t) <= p(t) in float64; the last position of a sequence finds the
//      first rejection L for both rules and writes every emitted token except
//      the draw;
//   3. float64 log-sum-exp of the draw rows of sequences that rejected (the
//      residual mixes p and q, so both must be exact to float64 precision);
//   4. the draw: float64 masses of each segment of the draw row (residual
//      max(p - q, 0), or p for the bonus token), then the last workgroup
//      picks the segment whose prefix crosses u * W and rescans it in id
//      order.
//
// Sampler-match ("speculative-acceptance.md", "The rules", the default rule
// at T > 0) replaces passes 2-4 by:
//   2. match pass, one workgroup per (position, segment): the masses of p
//      below the drafted token t and in all, and sum p*q (the rule's
//      acceptance probability, "Verifying the gain").  The fresh draw from p
//      lands on t iff mass(< t) <= u*W < mass(< t) + p(t); the masses come from
//      float32 terms, so a decision closer to a boundary than they resolve is
//      taken again with float64 terms over the row;
//   4. the draw at the first mismatch (or the bonus row), as above from p.
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
// SP: also sum p*q per position (the sampler-match acceptance probability,
// reported beside sum min(p, q) as "Verifying the gain before trusting a
// throughput number" prints both closed forms), one more FMA per element.
template <bool VEC, bool FILT, bool SP>
__global__ __launch_bounds__(NT) void coupling_kernel(SpecArgs a) {
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
  const bool bad = a.st_bad[trow] || a.st_bad[nT + drow];
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);

  // filtered rows: an element below its row's key floor has p (q) = 0
  const uint64_t kz = FILT ? a.kfl[trow] : 0ull, kd = FILT ? a.kfl[nT + drow] : 0ull;
  double tot = 0.0, tsp = 0.0;
  if (a.T > 0.0f && !bad) {
    const float c = a.lse_c;
    const double Lp = a.st_lse[trow] * (double)kLog2e, Lq = a.st_lse[nT + drow] * (double)kLog2e;
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
          float p = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gz[j].w[e]), c, -Lp_hi)) * fp;
          float q = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gd[j].w[e]), c, -Lq_hi)) * fq;
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
    for (int64_t t0 = e_tiles; t0 < e_full; t0 += (int64_t)NT * E) {
      Group gz[1], gd[1];
      load_tile<float, 1, VEC>(gz, zr, t0, e_full);
      load_tile<float, 1, VEC>(gd, dr, t0, e_full);
      pair(gz, gd, t0);
    }
    if (tid == 0)
      for (int64_t x = e_full; x < e_end; ++x) {
        float p = __builtin_amdgcn_exp2f(fmaf(zr[x], c, -Lp_hi)) * fp;
        float q = __builtin_amdgcn_exp2f(fmaf(dr[x], c, -Lq_hi)) * fq;
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
      const double Td = a.T;
      double pt = exp((double)zr[t] / Td - a.st_lse[trow]);
      double qt = exp((double)dr[t] / Td - a.st_lse[nT + drow]);
      if (FILT && comp_key(__float_as_uint(zr[t]), t) < kz) pt = 0.0;
      if (FILT && comp_key(__float_as_uint(dr[t]), t) < kd) qt = 0.0;
      flag = ((double)a.u_acc[pos] * qt <= pt) ? 1u : 0u;
    }
    st_dev(&a.acc[pos], flag);
    if (a.summin) st_dev(&a.summin[pos], bad ? __builtin_nanf("") : (float)tot);
    if (SP) st_dev(&a.sumprod[pos], bad ? __builtin_nanf("") : (float)tsp);
  }
  if (!last_done(sh, a.tk_seq + b, (uint32_t)G)) return;
  if (tid < G) sh.hist[tid] = ld_dev(&a.acc[b * G + tid]);
  __syncthreads();
  if (tid != 0) return;

  // Sequence decision.
  uint32_t* tm = a.tok_mrs + b * (G + 1);
  uint32_t* ta = a.tok_aa ? a.tok_aa + b * (G + 1) : nullptr;
  bool fail = a.st_bad[b * (G + 1) + G] != 0;
  for (int64_t q = 0; q < G; ++q) fail |= sh.hist[q] == 2u;
  for (int64_t q = 0; q <= G; ++q) {
    tm[q] = kFail;
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
  int64_t L = G;
  for (int64_t q = 0; q < G; ++q)
    if (sh.hist[q] == 0u) {
      L = q;
      break;
    }
  a.len_mrs[b] = (int32_t)L;
  for (int64_t q = 0; q < L; ++q) tm[q] = a.tokens[b * G + q];
  a.draw_L[b] = (int32_t)L;
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
    const float c = a.lse_c;
    const double Lp = a.st_lse[trow] * (double)kLog2e, Lq = a.st_lse[nT + drow] * (double)kLog2e;
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
          float p = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gz[j].w[e]), c, -Lp_hi)) * fp;
          float q = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(gd[j].w[e]), c, -Lq_hi)) * fq;
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
    for (int64_t t0 = e_tiles; t0 < e_full; t0 += (int64_t)NT * E) {
      Group gz[1], gd[1];
      load_tile<float, 1, VEC>(gz, zr, t0, e_full);  // past e_full: -inf, so p = q = 0
      load_tile<float, 1, VEC>(gd, dr, t0, e_full);
      pair(gz, gd, t0);
    }
    if (tid == 0)
      for (int64_t x = e_full; x < e_end; ++x) {
        float p = __builtin_amdgcn_exp2f(fmaf(zr[x], c, -Lp_hi)) * fp;
        float q = __builtin_amdgcn_exp2f(fmaf(dr[x], c, -Lq_hi)) * fq;
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
template <bool VEC>
__global__ __launch_bounds__(NT) void draw_lse_kernel(SpecArgs a) {
  constexpr int E = 4;
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const Item it = work_item(a.dS);  // the draw segments: few rows, many workgroups
  const int64_t item = it.row;  // b*2 + which
  const int seg = (int)it.seg;
  if (item >= a.B * 2) return;
  const int64_t b = item >> 1;
  const int which = (int)(item & 1);
  const int64_t G = a.gamma;
  const int32_t L = a.draw_L[b];
  if (L < 0 || L >= G) return;  // no residual draw for this sequence
  const int64_t nT = a.B * (G + 1);
  const int64_t srow = which == 0 ? b * (G + 1) + L : nT + b * G + L;
  const float* __restrict__ xr = which == 0 ? a.tgt + (b * (G + 1) + L) * a.ld_t : a.dft + (b * G + L) * a.ld_d;
  const double m = a.st_max[srow];
  const double Td = a.T, iT = 1.0 / Td;
  __shared__ double e2[64];
  init_e2(e2);
  const int64_t e_begin = (int64_t)seg * a.dseg, e_end = min(a.V, e_begin + a.dseg);
  double s = 0.0;
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  walk_groups<float, PG, VEC>(xr, e_begin, e_full, [&](const auto& g, int64_t) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
#pragma unroll
    for (int j = 0; j < NGP; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) s += exp_le0(((double)__uint_as_float(g[j].w[e]) - m) * iT, e2);
  });
  if (tid == 0)
    for (int64_t x = e_full; x < e_end; ++x) s += exp_le0(((double)xr[x] - m) * iT, e2);
  s = block_sum_f64(sh, s);
  if (a.dS > 1) {
    if (tid == 0) st_dev(&a.p_lse[item * a.dS + seg], s);
    if (!last_done(sh, a.tk_row + item, (uint32_t)a.dS)) return;
    s = merge_sum(sh, a.p_lse + item * a.dS, a.dS);
  }
  if (tid == 0) a.lse64[item] = m / Td + log(s);
}

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

// Chunk masses of segment [e_begin, e_end): each wave takes 4 chunks per
// step (16 loads per lane in flight), reduces each chunk's 256 weights (4 per
// lane) in float64, and writes the masses to `cm` (LDS) and `pc` (global,
// indexed from the segment's first chunk).  Returns the segment mass in
// thread 0: the in-order sum of its chunk masses.
template <typename DT>
__device__ double chunk_masses(const DrawSrc<DT>& r, int64_t e_begin, int64_t e_end, double* cm, double* pc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int CW = 4;  // chunks per wave per step
  const int nch = (int)((e_end - e_begin + kChunk - 1) / kChunk);
  for (int q0 = 0; q0 < nch; q0 += NWAVE * CW) {
    float zz[CW][4], dd[CW][4];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int q = q0 + wave * CW + j;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t x = e_begin + (int64_t)q * kChunk + lane * 4 + e;
        const bool in = q < nch && x < e_end;
        const int64_t xs = in ? x : e_begin;
        const float zx = r.zv(xs);
        const float dx = r.d ? r.d[xs] : 0.0f;
        zz[j][e] = in ? zx : -__builtin_inff();  // weight 0
        dd[j][e] = in ? dx : 0.0f;
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

// The draw itself (one workgroup): segment, then chunk, then element.  pw
// (LDS) holds the S segment masses, pc (global) the row's chunk masses.
// Returns the token in every thread; *W_out (thread 0) is the total mass.
template <typename DT>
__device__ uint32_t draw_pick(SelShared& sh, const DrawSrc<DT>& r, const double* pw, const double* pc, int S,
                              int64_t seg_len, double u, double* W_out) {
  const int tid = threadIdx.x;
  __shared__ double cm[kChunksPerSeg];
  __shared__ int s_seg, s_ch;
  __shared__ double s_in;
  __shared__ uint32_t s_tok;
  if (tid == 0) {
    double W = 0.0;
    for (int sg = 0; sg < S; ++sg) W += pw[sg];
    const double target = u * W;
    double cum = 0.0;
    int pick = -1;
    for (int sg = 0; sg < S; ++sg) {
      if (target < cum + pw[sg]) {
        pick = sg;
        break;
      }
      cum += pw[sg];
    }
    double tin = target - cum;
    if (pick < 0) {  // rounding at the very top: the last segment with mass
      for (int sg = S - 1; sg >= 0; --sg)
        if (pw[sg] > 0.0) {
          pick = sg;
          break;
        }
      if (pick < 0) pick = 0;
      tin = pw[pick];
    }
    s_seg = pick;
    s_in = tin;
    s_tok = kFail;
    *W_out = W;
  }
  __syncthreads();
  const int64_t e_begin = (int64_t)s_seg * seg_len, e_end = min(r.V, e_begin + seg_len);
  const int nch = (int)((e_end - e_begin + kChunk - 1) / kChunk);
  for (int q = tid; q < nch; q += NT) cm[q] = ld_dev(&pc[e_begin / kChunk + q]);
  __syncthreads();
  if (tid == 0) {
    const double tin = s_in;
    double cum = 0.0;
    int pick = -1;
    for (int q = 0; q < nch; ++q) {
      if (tin < cum + cm[q]) {
        pick = q;
        break;
      }
      cum += cm[q];
    }
    double t2 = tin - cum;
    if (pick < 0) {
      for (int q = nch - 1; q >= 0; --q)
        if (cm[q] > 0.0) {
          pick = q;
          break;
        }
      if (pick < 0) pick = 0;
      t2 = cm[pick];
    }
    s_ch = pick;
    s_in = t2;
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

__global__ __launch_bounds__(NT) void spec_draw_kernel(SpecArgs a) {
  __shared__ SelShared sh;
  __shared__ double cmw[kChunksPerSeg];
  const int tid = threadIdx.x;
  const Item it = work_item(a.dS);
  const int64_t b = it.row;
  const int seg = (int)it.seg;
  if (b >= a.B) return;
  const int64_t G = a.gamma;
  const int32_t L = a.draw_L[b];
  if (L < 0) return;
  __shared__ double e2[64];
  init_e2(e2);
  DrawSrc<float> r;
  r.T = a.T;
  r.iT = 1.0 / r.T;
  r.e2 = e2;
  r.V = a.V;
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
    r.lp = a.kfl ? a.st_lse[b * (G + 1) + L] : a.lse64[b * 2];
    r.lq = a.kfl ? a.st_lse[nT + b * G + L] : a.lse64[b * 2 + 1];
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
  const double ms = chunk_masses(r, e_begin, e_end, cmw, pc + e_begin / kChunk);
  if (tid == 0) st_dev(&a.p_w[b * a.dS + seg], ms);
  if (!last_done(sh, a.tk_draw + b, (uint32_t)a.dS)) return;
  __shared__ double pw[kMaxSegments];
  if (tid < a.dS) pw[tid] = ld_dev(&a.p_w[b * a.dS + tid]);
  __syncthreads();
  // Degenerate residual (p <= q everywhere): draw from p instead.
  __shared__ int s_degen;
  if (tid == 0) {
    double W = 0.0;
    for (int sg = 0; sg < a.dS; ++sg) W += pw[sg];
    s_degen = (r.d != nullptr && !(W > 0.0)) ? 1 : 0;
  }
  __syncthreads();
  if (s_degen) {
    r.d = nullptr;
    r.m = a.st_max[b * (G + 1) + L];
    for (int sg = 0; sg < a.dS; ++sg) {
      const int64_t eb = (int64_t)sg * a.dseg, ee = min(a.V, eb + a.dseg);
      const double m2 = chunk_masses(r, eb, ee, cmw, pc + eb / kChunk);
      if (tid == 0) pw[sg] = m2;
      __syncthreads();
    }
  }
  double W;
  const uint32_t tok = draw_pick(sh, r, pw, pc, a.dS, a.dseg, u, &W);
  if (tid == 0) (a.match ? a.tok_sm : a.tok_mrs)[b * (G + 1) + L] = tok;
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
  if (a.top_n_sigma > 0.0f) r.thr = r.m - (double)a.top_n_sigma * a.sigma[row];
  if (a.min_p > 0.0f) r.thr = fmax(r.thr, r.m + log((double)a.min_p));
  double* pc = a.p_c + row * a.nchunk;
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);
  const double ms = chunk_masses(r, e_begin, e_end, cmw, pc + e_begin / kChunk);
  if (tid == 0) st_dev(&a.p_w[row * a.S + seg], ms);
  if (!last_done(sh, a.tickets + row, (uint32_t)a.S)) return;
  __shared__ double pw[kMaxSegments];
  if (tid < a.S) pw[tid] = ld_dev(&a.p_w[row * a.S + tid]);
  __syncthreads();
  double W;
  const uint32_t tok = draw_pick(sh, r, pw, pc, a.S, a.seg_len, (double)a.u[row], &W);
  if (tid == 0) {
    a.out_token[row] = tok;
    if (a.out_logp) a.out_logp[row] = (float)(((double)r.zv(tok) - r.m) / r.T - log(W));
  }
}

template <bool VEC, bool FILT>
static void launch_coupling(bool sp, unsigned npos, const SpecArgs& a, hipStream_t s) {
  if (sp)
    hipLaunchKernelGGL((coupling_kernel<VEC, FILT, true>), dim3(npos), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((coupling_kernel<VEC, FILT, false>), dim3(npos), dim3(NT), 0, s, a);
}

hipError_t launch_spec(const SpecArgs& a, hipStream_t s) {
  const bool vec = a.vec_t && a.vec_d;
  const unsigned npos = (unsigned)(a.B * a.gamma * a.S);
  const bool sp = a.sumprod != nullptr;
  if (a.kfl) {
    if (vec)
      launch_coupling<true, true>(sp, npos, a, s);
    else
      launch_coupling<false, true>(sp, npos, a, s);
  } else {
    if (vec)
      launch_coupling<true, false>(sp, npos, a, s);
    else
      launch_coupling<false, false>(sp, npos, a, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.T == 0.0f) return e;
  if (a.kfl) {  // the filter pass already holds the exact lse of every row
    hipLaunchKernelGGL(spec_draw_kernel, dim3((unsigned)(a.B * a.dS)), dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  if (vec)
    hipLaunchKernelGGL(draw_lse_kernel<true>, dim3((unsigned)(a.B * 2 * a.dS)), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(draw_lse_kernel<false>, dim3((unsigned)(a.B * 2 * a.dS)), dim3(NT), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(spec_draw_kernel, dim3((unsigned)(a.B * a.dS)), dim3(NT), 0, s, a);
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
