// scan.hip -- one pass per row: first-maximum argmax, maximum, nonfinite
// latch and (optionally) log-sum-exp at a temperature.
//
// The pages reduce a row in two dispatches: 1,024-element chunks to
// per-chunk (value, index) partials, then the partials to one winner, with
// a strict greater-than so ties keep the lower index ("Chapter 21", sections
// 21.3-21.5 and Figure 21.1).  Here each workgroup streams a segment of the
// row with 16-byte loads, every lane keeps its own first maximum (its
// elements arrive in index order), the lanes' results are packed as
// (order-preserving key << 32 | ~index) so one unsigned max reduces them
// with the lower index winning ties, and the last workgroup of the row
// (atomic ticket) combines the segment partials -- one launch instead of
// two, and no read of a partial before it is visible.  A NaN or +inf
// element poisons the NaN-propagating running maximum, which latches the
// row to 0xFFFFFFFF as the greedy serving kernel does (section 21.4).
#include "device.hpp"
#include "internal.hpp"

namespace vsel {

constexpr int SG = 8;            // 16-byte groups per lane per tile
constexpr float kLazyScan = 64.0f; // the exp2 offset moves when a maximum passes it by this

template <typename DT, bool WANT_LSE, bool VEC, bool EXCL = false, bool MOM = false>
__global__ __launch_bounds__(NT) void scan_kernel(ScanArgs a) {
  constexpr int E = Elem<DT>::E;
  constexpr int64_t TILE = (int64_t)NT * SG * E;
  __shared__ SelShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows1 + a.rows2) return;
  const bool second = row >= a.rows1;
  const DT* __restrict__ xr = second ? reinterpret_cast<const DT*>(a.x2) + (row - a.rows1) * a.ld2
                                     : reinterpret_cast<const DT*>(a.x1) + row * a.ld1;
  const int64_t e_begin = (int64_t)seg * a.seg_len;
  const int64_t e_end = min(a.V, e_begin + a.seg_len);
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  const float c = a.lse_c;

  // First maximum without a search per group: each lane keeps its best
  // group (strictly greater, so the earliest of equal maxima -- a lane's
  // elements arrive in index order), that group's position and its words;
  // the first element equal to the maximum is found once, at the end.
  float best = -__builtin_inff();
  uint32_t bpos = 0, tail_idx = 0;
  bool from_tail = false;
  Group bw;
#pragma unroll
  for (int i = 0; i < 4; ++i) bw.w[i] = 0u;

  // Log-sum-exp with a lazy offset om (input units), as in the fused top-k
  // kernel: LS is the lane's sum of 2^((x - om) c) in float64; terms are
  // exp2(fma(x, c, noff)) with noff = -fl(om c), corrected by corr = 2^-delta
  // for that rounding when folded in; past |om| = 2^25 the lane takes exact
  // exp2((x - om) c) terms (huge).  A tile maximum above trig moves om.
  float lm = -__builtin_inff(), om = -__builtin_inff(), trig = -__builtin_inff(), noff = 0.0f, ls = 0.0f;
  double LS = 0.0, corr = 1.0;
  bool huge = false;
  auto set_offset = [&](float m) {
    LS = (om == -__builtin_inff()) ? 0.0 : LS * exp2_split(((double)om - (double)m) * (double)c);
    om = m;
    const float oc = m * c;
    noff = -oc;
    trig = m + kLazyScan / c;
    corr = exp2_split((double)oc - (double)m * (double)c);
    huge = !(__builtin_fabsf(m) <= 0x1p25f);
  };

  // Greedy serving variant ("Chapter 21", section 21.4): the request's
  // excluded ids are -inf inside the reduction only.  Each wave holds the
  // (at most 256) ids in four registers per lane; a tile tests them with one
  // range compare and a ballot each, and the lane holding an excluded
  // element replaces it in its registers before anything reads it.  A NaN
  // or +inf there keeps its value, so the row still fails closed.
  const int n_excl = EXCL ? a.n_excl : 0;
  uint32_t exid[kMaxExcluded / 64];
#pragma unroll
  for (int q = 0; q < kMaxExcluded / 64; ++q) {
    const int i = q * 64 + lane;
    exid[q] = (EXCL && i < n_excl) ? a.excl[i] : 0xFFFFFFFFu;
  }
  auto mask_bits = [&](uint32_t b) -> uint32_t {
    // the element's bits as float32 (bfloat16 widened); keep NaN and +inf
    const float x = __uint_as_float(E == 8 ? (b << 16) : b);
    const bool keep = (x != x) || x == __builtin_inff();
    return keep ? b : (E == 8 ? 0xFF80u : kNegInfBits);
  };
  auto exclude = [&](auto& g, uint32_t t0, uint32_t span) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
#pragma unroll
    for (int q = 0; q < kMaxExcluded / 64; ++q) {
      if (q * 64 >= n_excl) break;
      const uint32_t rel = exid[q] - t0;  // ids below t0 wrap past span
      uint64_t hits = __ballot(rel < span);
      while (hits) {
        const int bl = __builtin_ctzll(hits);
        hits &= hits - 1;
        const uint32_t er = (uint32_t)__builtin_amdgcn_readlane((int)rel, bl);
        const uint32_t gi = er / (uint32_t)E, el = er % (uint32_t)E;
        const uint32_t jj = gi / NT, owner = gi % NT;
        if ((uint32_t)tid == owner) {
#pragma unroll
          for (int j = 0; j < NGP; ++j) {
            if ((uint32_t)j != jj) continue;
            if constexpr (E == 8) {
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                if ((uint32_t)w != (el >> 1)) continue;
                const uint32_t word = g[j].w[w];
                if (el & 1u) g[j].w[w] = (word & 0xFFFFu) | (mask_bits(word >> 16) << 16);
                else g[j].w[w] = (word & 0xFFFF0000u) | mask_bits(word & 0xFFFFu);
              }
            } else {
#pragma unroll
              for (int w = 0; w < 4; ++w)
                if ((uint32_t)w == el) g[j].w[w] = mask_bits(g[j].w[w]);
            }
          }
        }
      }
    }
  };

  // Row moments (MOM): each lane's values above -inf shifted by its first
  // such value (in stream order), in float64, as the moments pass takes
  // them; the shift is settled once per group, in the groups a lane meets
  // before that value, and the count is an integer.
  uint32_t mcnt = 0;
  double mr = 0.0, ms1 = 0.0, ms2 = 0.0;
  auto mom_add = [&](const float (&x)[E]) {
    if constexpr (MOM) {
      if (mcnt == 0u) {
        float first = -__builtin_inff();
#pragma unroll
        for (int e = E - 1; e >= 0; --e) first = x[e] > -__builtin_inff() ? x[e] : first;
        if (first > -__builtin_inff()) mr = (double)first;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool ok = x[e] > -__builtin_inff();
        const double d = ok ? (double)x[e] - mr : 0.0;
        mcnt += ok ? 1u : 0u;
        ms1 += d;
        ms2 = fma(d, d, ms2);
      }
    }
  };

  auto group = [&](const Group& g, uint32_t pos) {
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = __uint_as_float(gbits<DT>(g, e));
    mom_add(x);
    float m0 = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) m0 = fmax_nan(m0, x[e]);
    const bool upd = m0 > best;
    best = upd ? m0 : best;
    bpos = upd ? pos : bpos;
#pragma unroll
    for (int i = 0; i < 4; ++i) bw.w[i] = upd ? g.w[i] : bw.w[i];
    if constexpr (WANT_LSE) {
      float acc = __builtin_amdgcn_exp2f(fmaf(x[0], c, noff));
#pragma unroll
      for (int e = 1; e < E; ++e) acc += __builtin_amdgcn_exp2f(fmaf(x[e], c, noff));
      ls += acc;
    }
    return m0;
  };

  // After a tile's terms are in ls: a lane whose tile maximum passed its
  // trigger moves its offset there; it, and a lane past the fast-path range,
  // recompute the tile's terms.
  auto lse_check = [&](auto& g, float tmax) {
    lm = fmax_nan(lm, tmax);
    if constexpr (WANT_LSE) {
      constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
      const bool up = tmax > trig && tmax < __builtin_inff();
      if (__ballot(up || huge)) {
        if (up) set_offset(tmax);
        if (up || huge) {
          auto fresh = [&](int j, float (&x)[E]) {
            uint32_t w0 = g[j].w[0], w1 = g[j].w[1], w2 = g[j].w[2], w3 = g[j].w[3];
            asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
            Group gf;
            gf.w[0] = w0; gf.w[1] = w1; gf.w[2] = w2; gf.w[3] = w3;
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = __uint_as_float(gbits<DT>(gf, e));
          };
          ls = 0.0f;
          if (huge) {
            for (int j = 0; j < NGP; ++j) {
              float x[E];
              fresh(j, x);
#pragma unroll
              for (int e = 0; e < E; ++e) ls += __builtin_amdgcn_exp2f((x[e] - om) * c);
            }
          } else {
            for (int j = 0; j < NGP; ++j) {
              float x[E];
              fresh(j, x);
#pragma unroll
              for (int e = 0; e < E; ++e) ls += __builtin_amdgcn_exp2f(fmaf(x[e], c, noff));
            }
          }
        }
      }
    }
  };
  auto fold = [&]() {
    if constexpr (WANT_LSE) {
      LS += huge ? (double)ls : (double)ls * corr;
      ls = 0.0f;
    }
  };
  // Before the first tile's terms: start the offset at the lane's maximum
  // of that tile (the asm keeps these unpacked values from being shared
  // with the pass that follows).
  auto seed = [&](auto& g) {
    if constexpr (WANT_LSE) {
      constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
      float m = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < NGP; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmax_nan(m, __uint_as_float(gbits<DT>(g[j], e)));
#pragma unroll
      for (int j = 0; j < NGP; ++j) asm volatile("" : "+v"(g[j].w[0]), "+v"(g[j].w[1]), "+v"(g[j].w[2]), "+v"(g[j].w[3]));
      if (m > -__builtin_inff() && m < __builtin_inff()) set_offset(m);
    }
  };

  const int64_t e_tiles = e_begin + (e_full - e_begin) / TILE * TILE;
  bool first = true;
  // Fair progress, as in the per-wave top-k kernel: a wave starts at the
  // highest issue priority and drops one level per quarter of its tiles, so
  // waves that are ahead yield to those behind (a younger workgroup's
  // quarters end one tile later per step of age).
  const uint32_t ntiles = (uint32_t)((e_tiles - e_begin) / TILE);
  const uint32_t age = (blockIdx.x * 4u) / gridDim.x;
  const uint32_t q1 = ntiles / 4 + age, q2 = ntiles / 2 + age, q3 = ntiles - ntiles / 4 + age;
  __builtin_amdgcn_s_setprio(3);
  uint32_t tix = 0;
  for (int64_t t0 = e_begin; t0 < e_tiles; t0 += TILE) {
    ++tix;
    if (tix == q1) __builtin_amdgcn_s_setprio(2);
    else if (tix == q2) __builtin_amdgcn_s_setprio(1);
    else if (tix == q3) __builtin_amdgcn_s_setprio(0);
    Group g[SG];
    if constexpr (VEC) load_tile_buf<DT, SG>(g, xr + t0);
    else load_tile_full<DT, SG, false>(g, xr + t0);
    if constexpr (EXCL) exclude(g, (uint32_t)t0, (uint32_t)TILE);
    if (first) {
      seed(g);
      first = false;
    }
    float tmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < SG; ++j) tmax = fmax_nan(tmax, group(g[j], (uint32_t)t0 + (uint32_t)(j * NT + tid) * E));
    if constexpr (WANT_LSE) asm volatile("" ::"v"(ls), "v"(tmax));
    lse_check(g, tmax);
    fold();
  }
  // the segment's last partial tile, its loads issued together (groups past
  // e_full read as -inf)
  if (e_tiles < e_full) {
    Group g[SG];
    load_tile<DT, SG, VEC>(g, xr, e_tiles, e_full);
    if constexpr (EXCL) exclude(g, (uint32_t)e_tiles, (uint32_t)(e_full - e_tiles));
    if (first) {
      seed(g);
      first = false;
    }
    float tmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < SG; ++j) tmax = fmax_nan(tmax, group(g[j], (uint32_t)e_tiles + (uint32_t)(j * NT + tid) * E));
    if constexpr (WANT_LSE) asm volatile("" ::"v"(ls), "v"(tmax));
    lse_check(g, tmax);
    fold();
  }
  // the row's last few elements (fewer than one group): one lane, after
  // wave 0 marks which of them are excluded
  uint32_t tail_ex = 0;
  if (EXCL && e_full < e_end && wave == 0 && n_excl > 0) {
#pragma unroll
    for (int q = 0; q < kMaxExcluded / 64; ++q) {
      const uint32_t rel = exid[q] - (uint32_t)e_full;
      const uint64_t hits = __ballot(rel < (uint32_t)(e_end - e_full));
      uint64_t h = hits;
      while (h) {
        const int bl = __builtin_ctzll(h);
        h &= h - 1;
        tail_ex |= 1u << (uint32_t)__builtin_amdgcn_readlane((int)rel, bl);
      }
    }
  }
  if (e_full < e_end && tid == 0) {
    for (int64_t i = e_full; i < e_end; ++i) {
      const uint32_t braw = gbits_at<DT>(xr, i);
      const bool ex = (tail_ex >> (uint32_t)(i - e_full)) & 1u;
      const float xo = __uint_as_float(braw);
      const float x = (ex && !(xo != xo || xo == __builtin_inff())) ? -__builtin_inff() : xo;
      if (x > best) {
        best = x;
        tail_idx = (uint32_t)i;
        from_tail = true;
      }
      lm = fmax_nan(lm, x);
      if constexpr (MOM) {
        float x1[E];
#pragma unroll
        for (int e = 0; e < E; ++e) x1[e] = e == 0 ? x : -__builtin_inff();
        mom_add(x1);
      }
      if constexpr (WANT_LSE) {
        if (x > trig && x < __builtin_inff()) set_offset(x);
        LS += huge ? (double)__builtin_amdgcn_exp2f((x - om) * c)
                   : (double)__builtin_amdgcn_exp2f(fmaf(x, c, noff)) * corr;
      }
    }
  }
  // the lane's first maximum inside its best group
  uint32_t bidx = tail_idx;
  if (!from_tail) {
    uint32_t f = E - 1;
#pragma unroll
    for (int e = E - 2; e >= 0; --e) f = (__uint_as_float(gbits<DT>(bw, e)) == best) ? (uint32_t)e : f;
    bidx = bpos + f;
  }

  uint64_t P = (best > -__builtin_inff()) ? (((uint64_t)fkey(__float_as_uint(best)) << 32) | (uint32_t)~bidx) : 0ull;
  P = wave_max_u64(P);
  if (lane == 0) sh.wk[wave] = P;
  LSE r{lm, 0.0};
  if constexpr (WANT_LSE) {
    if (lm != lm || lm == __builtin_inff()) r.s = __builtin_nan("");
    else if (lm != -__builtin_inff()) r.s = LS * exp2_split(((double)om - (double)lm) * (double)c);
  }
  r = block_lse(r, c, sh.wm, sh.ws);  // its barriers also publish sh.wk
  P = sh.wk[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) P = sh.wk[q] > P ? sh.wk[q] : P;

  // Moments (MOM): the lanes folded per wave, then the waves in order, then
  // (below) the segments, each in a fixed order.
  __shared__ double s_mom[3 * NWAVE];
  auto fold_waves = [&](Mom v) {
    v = wave_mom(v);
    __syncthreads();
    if (lane == 0) {
      s_mom[wave] = v.n;
      s_mom[NWAVE + wave] = v.mean;
      s_mom[2 * NWAVE + wave] = v.m2;
    }
    __syncthreads();
    Mom w{0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) w = mom_merge(w, Mom{s_mom[q], s_mom[NWAVE + q], s_mom[2 * NWAVE + q]});
    return w;
  };
  Mom mv{0.0, 0.0, 0.0};
  if constexpr (MOM) {
    const double mn = (double)mcnt;
    Mom v{mn, 0.0, 0.0};
    if (mn > 0.0) v = Mom{mn, mr + ms1 / mn, ms2 - ms1 * ms1 / mn};
    mv = fold_waves(v);
  }

  if (a.S > 1) {
    const int64_t slot = row * a.S + seg;
    if (tid == 0) {
      st_dev(&a.p_key[slot], P);
      st_dev(&a.p_m[slot], r.m);
      st_dev(&a.p_s[slot], r.s);
      if constexpr (MOM) {
        st_dev(&a.m_n[slot], mv.n);
        st_dev(&a.m_mean[slot], mv.mean);
        st_dev(&a.m_m2[slot], mv.m2);
      }
    }
    if (!last_done(sh, a.tickets + row, (uint32_t)a.S)) return;
    const int64_t s0 = row * a.S;
    // this thread's segment's moments, loaded with the partials below
    Mom ms{0.0, 0.0, 0.0};
    if constexpr (MOM) {
      if (tid < a.S) ms = Mom{ld_dev(&a.m_n[s0 + tid]), ld_dev(&a.m_mean[s0 + tid]), ld_dev(&a.m_m2[s0 + tid])};
    }
    merge_key_lse(sh, a.p_key + s0, a.p_m + s0, a.p_s + s0, a.S, c, P, r);
    if constexpr (MOM) mv = fold_waves(ms);
  }
  if (tid != 0) return;
  if constexpr (MOM) a.sigma[row] = mv.n > 0.0 ? sqrt(fmax(mv.m2, 0.0) / mv.n) : 0.0;

  const bool bad = (r.m != r.m) || (r.m == __builtin_inff());
  const bool none = bad || P == 0;
  const uint32_t idx = none ? kFail : ~(uint32_t)P;
  if (a.out_idx) a.out_idx[row] = idx;
  if (a.out_status) a.out_status[row] = bad ? 1u : (P == 0 ? 2u : 0u);
  if (a.out_val)
    a.out_val[row] = bad ? __builtin_nanf("") : (P == 0 ? -__builtin_inff() : __uint_as_float(gbits_at<DT>(xr, idx)));
  if (a.out_logp0) a.out_logp0[row] = none ? __builtin_nanf("") : 0.0f;
  if (a.st_amax) a.st_amax[row] = idx;
  if (a.st_max) a.st_max[row] = r.m;
  if (a.st_bad) a.st_bad[row] = none ? 1u : 0u;
  if (a.st_lse)
    a.st_lse[row] = bad ? __builtin_nan("") : (r.m == -__builtin_inff() ? -__builtin_inf() : (double)r.m / a.T + log(r.s));
}

template <typename DT, bool L>
static hipError_t go(const ScanArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows1 + a.rows2) * a.S));
  // both row sets must take the vector path for the VEC kernel
  const bool vec = a.vec1 && (a.rows2 == 0 || a.vec2);
  if constexpr (!L) {
    if (a.n_excl > 0) {
      if (vec)
        hipLaunchKernelGGL((scan_kernel<DT, false, true, true>), grid, dim3(NT), 0, s, a);
      else
        hipLaunchKernelGGL((scan_kernel<DT, false, false, true>), grid, dim3(NT), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (!L) {
    if (a.sigma) {  // the row moments in the same pass
      if (vec)
        hipLaunchKernelGGL((scan_kernel<DT, false, true, false, true>), grid, dim3(NT), 0, s, a);
      else
        hipLaunchKernelGGL((scan_kernel<DT, false, false, false, true>), grid, dim3(NT), 0, s, a);
      return hipGetLastError();
    }
  }
  if (vec)
    hipLaunchKernelGGL((scan_kernel<DT, L, true>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((scan_kernel<DT, L, false>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan(int dtype, bool want_lse, const ScanArgs& a, hipStream_t s) {
  if (dtype == 0) return want_lse ? go<float, true>(a, s) : go<float, false>(a, s);
  return want_lse ? go<uint16_t, true>(a, s) : go<uint16_t, false>(a, s);
}

template <typename DT, bool L>
static int occ() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_kernel<DT, L, true>, NT, 0) != hipSuccess) return 0;
  return n;
}

int scan_blocks_per_cu(int dtype, bool want_lse) {
  if (dtype == 0) return want_lse ? occ<float, true>() : occ<float, false>();
  return want_lse ? occ<uint16_t, true>() : occ<uint16_t, false>();
}

}  // namespace vsel
