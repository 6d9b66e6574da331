// topk.hip -- fused per-row top-k + argmax + log-sum-exp (and the sampling
// tail), one pass over the row.
//
// The device-side top_k + get_rows of llama.cpp PR #49 ("Change") keeps only
// k candidates per row on the way off the device.  Here one workgroup streams
// a segment of a row from HBM once, in tiles of 8 x 16-byte loads per lane,
// the next tile's loads in flight while the current one is processed:
//   * online log-sum-exp: one FMA + one exp2 + one add per element, float32
//     inside a tile, float64 across tiles, waves and segments;
//   * exact top-k by composite key (value desc, id asc).  An element can only
//     matter if it reaches T, a lower bound of the segment's k-th largest
//     composite key.  Each 16-byte group is tested once through its maximum;
//     a wave compacts its groups that reach T into a per-wave LDS staging list
//     (ballot + mbcnt), and its lanes then open the staged groups together and
//     append qualifying elements to the workgroup's LDS candidate buffer.  On
//     the first tile T comes from the lane maxima (the ceil(k/4)-th largest
//     lane maximum of each wave, minimum over the waves: at least k distinct
//     elements reach it); when the buffer grows past a few k records, a radix
//     select shrinks it to its k largest and raises T to their k-th key;
//   * at the end the buffer is cut to k records (segments of a row merge in
//     the row's last workgroup through an atomic ticket), the winners are
//     ordered by rank and written with their own element bits, the argmax is
//     the first winner and the log-sum-exp is finished in float64.
// The first-maximum rule of "Chapter 21", section 21.3, is the top-1 of the
// same order, so the argmax comes out of the selection for free.
#include "device.hpp"
#include "internal.hpp"

namespace vsel {

constexpr int TG = kTopkGroups;     // 16-byte groups per lane per tile
constexpr uint32_t kRankMax = 256;  // winners ordered by rank up to this many

constexpr uint32_t kStage = 128;    // staged groups per wave per tile

struct WaveStage {
  uint32_t w[kStage][4];
  uint32_t e0[kStage];
};

// Append one candidate to the workgroup buffer (or flag the overflow).
template <int CAP>
__device__ __forceinline__ void append(SelShared& sh, uint64_t* key, uint32_t* bits, uint64_t K, uint32_t b) {
  const uint32_t pos = atomicAdd(&sh.cnt, 1u);
  if (pos < (uint32_t)CAP) {
    key[pos] = K;
    bits[pos] = b;
  } else {
    sh.overflow = 1u;
  }
}

template <typename DT, bool WANT_LSE, int CAP, bool VEC>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  constexpr int E = Elem<DT>::E;
  __shared__ uint64_t s_key[CAP];
  __shared__ uint32_t s_bits[CAP];
  __shared__ __attribute__((aligned(16))) WaveStage stg[NWAVE];
  __shared__ SelShared sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  const DT* __restrict__ xr = reinterpret_cast<const DT*>(a.x) + row * a.ld;
  const int64_t e_begin = (int64_t)seg * a.seg_len;
  const int64_t e_end = min(a.V, e_begin + a.seg_len);
  const uint32_t k = (uint32_t)a.k;
  // whole groups; the row's ragged tail (fewer than E elements) is added at the end
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  const uint32_t e_full32 = (uint32_t)e_full;
  const float c = kLog2e;  // log-sum-exp at temperature 1
  // Shrink the buffer once it holds this many records (room for k more is
  // always kept, which the overflow path needs).
  const uint32_t select_at = min(max(4u * k, 512u), (uint32_t)CAP - k);

  if (tid == 0) {
    sh.cnt = 0;
    sh.overflow = 0;
  }
  __syncthreads();

  uint64_t T = 1;     // lower bound of the segment's k-th largest composite key
  uint32_t nbuf = 0;  // records in the buffer at the start of a tile
  LSE st{-__builtin_inff(), 0.0};

  // Open this wave's staged groups with all lanes: append every element that
  // reaches the threshold to the workgroup buffer.
  auto flush = [&](uint32_t sn, uint64_t thr, float tf) {
    for (uint32_t q = lane; q < sn; q += 64) {
      Group gg;
#pragma unroll
      for (int i = 0; i < 4; ++i) gg.w[i] = stg[wave].w[q][i];
      const uint32_t e0 = stg[wave].e0[q];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t b = gbits<DT>(gg, e);
        if (__uint_as_float(b) >= tf && e0 + e < e_full32) {
          const uint64_t K = comp_key(b, e0 + e);
          if (K >= thr) append<CAP>(sh, s_key, s_bits, K, b);
        }
      }
    }
  };

  auto process = [&](const auto& g, int64_t t0) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
    constexpr int TILEP = NT * NGP * E;
    // Per group: its maximum (for the candidate test), then -- with the
    // lane's running maximum mt -- its exp2 terms.  The tile's float32 sum
    // stile is folded into the float64 lane sum at the end of the tile.
    float gm[NGP];
    float tmax = -__builtin_inff();
    // exponents as (x - ob) * c with the offset ob in input units: exact for
    // the maximum itself at any magnitude (x * c - ob * c would carry the
    // rounding of both products)
    float mt = st.m, ob = 0.0f, stile = 0.0f;
    if constexpr (WANT_LSE) ob = (mt == -__builtin_inff()) ? 0.0f : mt;
#pragma unroll
    for (int j = 0; j < NGP; ++j) {
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __uint_as_float(gbits<DT>(g[j], e));
      float m0 = x[0];
#pragma unroll
      for (int e = 1; e < E; ++e) m0 = fmax_nan(m0, x[e]);
      gm[j] = m0;
      tmax = fmax_nan(tmax, m0);
      if constexpr (WANT_LSE) {
        const float mn = fmax_nan(mt, m0);
        if (!(mn == mt)) {  // the running maximum moved (or became NaN)
          const float ms = (mn == -__builtin_inff()) ? 0.0f : mn;
          stile *= __builtin_amdgcn_exp2f((mt - ms) * c);
          ob = ms;
          mt = mn;
        }
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc += __builtin_amdgcn_exp2f((x[e] - ob) * c);
        stile += acc;
      }
    }
    if constexpr (WANT_LSE) {
      // Finish the exp2 terms here, before the staging below: otherwise the
      // compiler sinks them past it and keeps the whole tile unpacked.
      asm volatile("" ::"v"(stile), "v"(mt));
      // fold: st.s is relative to st.m, stile to mt >= st.m
      // st.m < mt here unless equal; an empty state (st.m = -inf) scales to 0
      const double scale = (st.m == mt) ? 1.0 : (double)__builtin_amdgcn_exp2f((st.m - mt) * c);
      st.s = st.s * scale + (double)stile;
      st.m = mt;
    } else {
      st.m = fmax_nan(st.m, tmax);
    }

    // First tile: T from the lane maxima (needs k <= 4 waves x 64 lanes).
    if (t0 == e_begin && k <= (uint32_t)NWAVE * 64u) {
      const bool real = t0 + (int64_t)tid * E < e_full;
      const uint32_t lk = real ? fkey(__float_as_uint(tmax)) : 0u;
      const uint32_t kw = (k + NWAVE - 1) / NWAVE;
      uint32_t tw = 0;
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = tw | (1u << b);
        if ((uint32_t)__popcll(__ballot(lk >= cand)) >= kw) tw = cand;
      }
      if (lane == 0) sh.wtau[wave] = tw;
      __syncthreads();
      uint32_t tau = sh.wtau[0];
#pragma unroll
      for (int q = 1; q < NWAVE; ++q) tau = min(tau, sh.wtau[q]);
      const uint64_t Tn = (uint64_t)tau << 32;
      if (Tn > T) T = Tn;
    }

    // Stage this wave's groups that reach T, then open them with all lanes.
    // More than kStage staged groups in one wave sends the tile down the
    // overflow path below.
    const float tf = thr_float(T);
    const uint32_t cnt0 = nbuf;
    uint32_t sn = 0;
#pragma unroll
    for (int j = 0; j < NGP; ++j) {
      const bool pass = gm[j] >= tf;
      const uint64_t m = __ballot(pass);
      if (m) {
        const uint32_t p =
            sn + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (pass && p < kStage) {
#pragma unroll
          for (int i = 0; i < 4; ++i) stg[wave].w[p][i] = g[j].w[i];
          stg[wave].e0[p] = (uint32_t)t0 + (uint32_t)(j * NT + tid) * E;
        }
        sn += (uint32_t)__popcll(m);
      }
    }
    if (sn > kStage) {
      if (lane == 0) sh.overflow = 1u;
    } else {
      flush(sn, T, tf);
    }
    __syncthreads();

    if (sh.overflow) {
      // Too many candidates in this tile (buffer or staging full): drop its
      // appends and extract the tile again from memory.  If its elements at
      // or above T do not fit, first raise T to the tile's own k-th largest
      // key (exact radix select over the tile): then at most k are added.
      __syncthreads();
      if (tid == 0) {
        sh.cnt = cnt0;
        sh.overflow = 0;
        sh.cnt2 = 0;
      }
      __syncthreads();
      const int64_t t_end = min(e_full, t0 + (int64_t)TILEP);
      const uint64_t Tlow = T;
      uint32_t mine = 0;
      for (int64_t i = t0 + tid; i < t_end; i += NT) mine += comp_key(gbits_at<DT>(xr, i), (uint32_t)i) >= Tlow ? 1u : 0u;
      atomicAdd(&sh.cnt2, mine);
      __syncthreads();
      if (sh.cnt2 > (uint32_t)CAP - cnt0) {  // then it holds more than k keys >= Tlow
        const uint64_t Tt = radix_select(sh, k, [&](auto f) {
          for (int64_t i = t0 + tid; i < t_end; i += NT) {
            const uint64_t K = comp_key(gbits_at<DT>(xr, i), (uint32_t)i);
            if (K >= Tlow) f(K);
          }
        });
        if (Tt > T) T = Tt;
      }
      const float tf2 = thr_float(T);
      for (int64_t i = t0 + tid; i < t_end; i += NT) {
        const uint32_t b = gbits_at<DT>(xr, i);
        if (__uint_as_float(b) >= tf2) {
          const uint64_t K = comp_key(b, (uint32_t)i);
          if (K >= T) append<CAP>(sh, s_key, s_bits, K, b);
        }
      }
      __syncthreads();
    }
    nbuf = sh.cnt;
    if (nbuf > select_at) {
      T = select_compact<CAP>(sh, s_key, s_bits, nbuf, k);
      nbuf = k;
    }
  };

  walk_groups<DT, TG, VEC>(xr, e_begin, e_full, process);
  if (e_full < e_end) {
    // The row's last few elements (fewer than one group): one lane.  The
    // buffer always has room for them (at most CAP - k records are kept).
    if (tid == 0) {
      for (int64_t i = e_full; i < e_end; ++i) {
        const uint32_t b = gbits_at<DT>(xr, i);
        const float x = __uint_as_float(b);
        if constexpr (WANT_LSE) {
          const float mn = fmax_nan(st.m, x);
          const float ms = (mn == -__builtin_inff()) ? 0.0f : mn;
          const double scale = (st.m == mn) ? 1.0 : (double)__builtin_amdgcn_exp2f((st.m - ms) * c);
          st.s = st.s * scale + (double)__builtin_amdgcn_exp2f((x - ms) * c);
          st.m = mn;
        } else {
          st.m = fmax_nan(st.m, x);
        }
        const uint64_t K = comp_key(b, (uint32_t)i);
        if (K >= T) append<CAP>(sh, s_key, s_bits, K, b);
      }
    }
    __syncthreads();
    nbuf = sh.cnt;
  }

  uint32_t n = nbuf;
  if (n > k) {
    select_compact<CAP>(sh, s_key, s_bits, n, k);
    n = k;
  }

  // Segment log-sum-exp state.
  LSE r = wave_lse(st, c);
  if (lane == 0) {
    sh.wm[wave] = r.m;
    sh.ws[wave] = r.s;
  }
  __syncthreads();
  r = LSE{sh.wm[0], sh.ws[0]};
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) r = lse_merge(r, LSE{sh.wm[q], sh.ws[q]}, c);

  if (a.S > 1) {
    const int64_t slot = row * a.S + seg;
    for (uint32_t i = tid; i < n; i += NT) {
      st_dev(&a.rec_key[slot * k + i], s_key[i]);
      st_dev(&a.rec_bits[slot * k + i], s_bits[i]);
    }
    if (tid == 0) {
      st_dev(&a.rec_cnt[slot], n);
      st_dev(&a.p_m[slot], r.m);
      st_dev(&a.p_s[slot], r.s);
    }
    if (!last_done(sh, a.tickets + row, (uint32_t)a.S)) return;
    const int64_t s0 = row * a.S;
    // record counts of all segments at once (in flight with the (max, sum)
    // partials), then their offsets (wave 0)
    const uint32_t cnt_t = tid < a.S ? ld_dev(&a.rec_cnt[s0 + tid]) : 0u;
    uint64_t unusedP;
    merge_key_lse(sh, nullptr, a.p_m + s0, a.p_s + s0, a.S, c, unusedP, r);
    if (tid < a.S) sh.hist[tid] = cnt_t;
    __syncthreads();
    if (tid < 64) {
      uint32_t cv[4], loc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cv[q] = (4 * tid + q < a.S) ? sh.hist[4 * tid + q] : 0u;
        loc += cv[q];
      }
      uint32_t run = wave_incl_scan_u32(loc, tid) - loc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (4 * tid + q < a.S) sh.hist[4 * tid + q] = run;
        run += cv[q];
      }
      if (tid == 63) sh.cnt2 = run;
    }
    __syncthreads();
    n = sh.cnt2;
    // every record of the row in rounds of loads: record f of the
    // concatenation is record f - off[sg] of segment sg (sg found by a binary
    // search of the offsets), kMergeQ per thread in flight at once
    constexpr int kMergeQ = 4;
    for (uint32_t f0 = 0; f0 < n; f0 += NT * kMergeQ) {
      uint64_t v[kMergeQ];
      uint32_t vb[kMergeQ];
#pragma unroll
      for (int q = 0; q < kMergeQ; ++q) {
        const uint32_t f = f0 + (uint32_t)(q * NT) + tid;
        if (f < n) {
          int lo = 0, hi = a.S - 1;  // the last segment whose offset is <= f
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.hist[mid] <= f) lo = mid;
            else hi = mid - 1;
          }
          const int64_t src = (s0 + lo) * k + (f - sh.hist[lo]);
          v[q] = ld_dev(&a.rec_key[src]);
          vb[q] = ld_dev(&a.rec_bits[src]);
        }
      }
#pragma unroll
      for (int q = 0; q < kMergeQ; ++q) {
        const uint32_t f = f0 + (uint32_t)(q * NT) + tid;
        if (f < n) {
          s_key[f] = v[q];
          s_bits[f] = vb[q];
        }
      }
    }
    __syncthreads();
    if (n > k) {
      select_compact<CAP>(sh, s_key, s_bits, n, k);
      n = k;
    }
  }

  // Order the winners (value desc, id asc): by rank into the upper half of
  // the buffer when there are few, else an in-place bitonic sort.
  uint64_t* okey = s_key;
  uint32_t* obits = s_bits;
  if (n <= kRankMax) {
    okey = s_key + CAP / 2;
    obits = s_bits + CAP / 2;
    for (uint32_t i = tid; i < n; i += NT) {
      const uint64_t K = s_key[i];
      uint32_t r0 = 0;
      for (uint32_t j = 0; j < n; ++j) r0 += s_key[j] > K ? 1u : 0u;
      okey[r0] = K;
      obits[r0] = s_bits[i];
    }
    __syncthreads();
  } else {
    sort_desc<CAP>(s_key, s_bits, n);
  }

  const bool bad = (r.m != r.m) || (r.m == __builtin_inff());
  const bool none = bad || r.m == -__builtin_inff();
  if (a.mode == 0) {
    for (uint32_t j = tid; j < k; j += NT) {
      a.out_ids[row * k + j] = bad ? kFail : ~(uint32_t)okey[j];
      a.out_vals[row * k + j] = bad ? __builtin_nanf("") : __uint_as_float(obits[j]);
    }
    if (tid == 0) {
      if (a.out_argmax) a.out_argmax[row] = none ? kFail : ~(uint32_t)okey[0];
      if (a.out_lse)
        a.out_lse[row] = bad ? __builtin_nanf("")
                             : (r.m == -__builtin_inff() ? -__builtin_inff() : (float)((double)r.m + log(r.s)));
    }
  } else {
    // the sampler chain; scratch in the halves of the buffers the winners
    // left free and in the staging area
    uint32_t tok = kFail;
    float lp = __builtin_nanf("");
    if (!none && n > 0) {
      double* E = reinterpret_cast<double*>(okey == s_key ? s_key + CAP / 2 : s_key);
      uint32_t* LIST = obits == s_bits ? s_bits + CAP / 2 : s_bits;
      // the typicality scores after E in the free half when both fit there
      // (up to 1,024 candidates in the large buffer), else in the staging area
      const bool in_half = 2 * n <= (uint32_t)(CAP / 2);
      double* Sc = in_half ? E + n : reinterpret_cast<double*>(&stg[0]);
      uint32_t* ORD = in_half ? &stg[0].w[0][0] : &stg[1].w[0][0];
      const ChainParams cp{a.temperature, a.top_p,  a.top_n_sigma, a.typical_p, a.min_p,
                           a.mode == 2 ? a.out_kfl + row : nullptr, a.mode == 2 ? a.out_lse_f + row : nullptr};
      chain_tail(okey, obits, n, cp, a.sigma ? a.sigma[row] : 0.0, a.u ? a.u[row] : 0.0f, E, Sc, ORD, LIST, &tok,
                 &lp);
    }
    if (tid == 0) {
      if (a.mode == 1) {
        a.out_token[row] = tok;
        if (a.out_logp) a.out_logp[row] = lp;
      } else if (none || n == 0) {  // (the caller fails such rows closed)
        a.out_kfl[row] = 0ull;
        a.out_lse_f[row] = __builtin_nan("");
      }
    }
  }
}

template <typename DT, bool L, int CAP>
static hipError_t go(const TopkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.S));
  if (a.vec)
    hipLaunchKernelGGL((topk_kernel<DT, L, CAP, true>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((topk_kernel<DT, L, CAP, false>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(int dtype, bool want_lse, int cap, const TopkArgs& a, hipStream_t s) {
  if (dtype == 0) {
    if (cap <= kCapSmall) return want_lse ? go<float, true, kCapSmall>(a, s) : go<float, false, kCapSmall>(a, s);
    return want_lse ? go<float, true, kCapLarge>(a, s) : go<float, false, kCapLarge>(a, s);
  }
  if (cap <= kCapSmall) return want_lse ? go<uint16_t, true, kCapSmall>(a, s) : go<uint16_t, false, kCapSmall>(a, s);
  return want_lse ? go<uint16_t, true, kCapLarge>(a, s) : go<uint16_t, false, kCapLarge>(a, s);
}

template <typename DT, bool L, int CAP>
static int occ() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, topk_kernel<DT, L, CAP, true>, NT, 0) != hipSuccess) return 0;
  return n;
}

int topk_blocks_per_cu(int dtype, bool want_lse, int cap) {
  if (dtype == 0) {
    if (cap <= kCapSmall) return want_lse ? occ<float, true, kCapSmall>() : occ<float, false, kCapSmall>();
    return want_lse ? occ<float, true, kCapLarge>() : occ<float, false, kCapLarge>();
  }
  if (cap <= kCapSmall) return want_lse ? occ<uint16_t, true, kCapSmall>() : occ<uint16_t, false, kCapSmall>();
  return want_lse ? occ<uint16_t, true, kCapLarge>() : occ<uint16_t, false, kCapLarge>();
}

}  // namespace vsel
