// topk_wave.hip -- fused per-row top-k + argmax + log-sum-exp (and the
// sampling tail) for k <= 128 on 16-byte-aligned rows, one pass over the row.
//
// Same result as topk_kernel; a different schedule.  The selection of PR #49
// ("Change": top_k + get_rows on each device's share) is fused with the
// argmax and the log-sum-exp, and the four waves of a workgroup filter their
// share of each tile independently, with no workgroup barrier while the row
// streams:
//   * log-sum-exp with a lazy offset: every element costs one FMA, one exp2
//     and one add against the lane's current offset, and the offset moves
//     (rescaling the lane's sums) only when a group maximum passes it by 2^64
//     -- the first group, and then almost never;
//   * each 16-byte group is tested once through its maximum against the
//     wave's threshold T (a lower bound of the segment's k-th largest
//     composite key); the wave compacts its passing groups into an LDS
//     staging list (ballot + mbcnt) and, every 64 staged groups, opens them
//     and appends the elements that reach T to its own LDS candidate list;
//   * a wave-level radix select cuts the list to k and raises T whenever the
//     list grows past a few k records;
//   * at the segment's end the four lists merge (workgroup select), segments
//     of a row merge in the row's last workgroup, and the winners are written
//     in (value desc, id asc) order.  A record is only its composite key; the
//     value comes back from the key, except for +-0 winners whose sign bit
//     the key folds away: those are read again from the row.
// The first tile's threshold is the one workgroup-wide step: the
// ceil(k/4)-th largest lane maximum of each wave, minimum over the waves,
// so at least k distinct elements reach it.
#include "device.hpp"
#include "internal.hpp"

namespace vsel {

constexpr int WTG = kTopkGroups;      // 16-byte groups per lane per tile
constexpr uint32_t kWCap = 512;       // candidate records per wave
constexpr uint32_t kWStage = 128;     // staged groups per wave
constexpr uint32_t kFlushAt = 64;     // open the staged groups at a tile end from this many
constexpr float kLazyLog2 = 64.0f;    // the exp2 offset moves when a maximum passes it by this
constexpr uint32_t kRank = NT;
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
        // records ordered by rank directly, one per thread

struct WaveArea {
  uint32_t w[kWStage][4];
  uint32_t e0[kWStage];
  uint32_t hist[256];
};

// Order the wave's LDS accesses around cross-lane communication (the LDS
// unit executes one wave's operations in order; this keeps the compiler from
// moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Threshold with exactly `rank` of the n > rank distinct keys wb[0..n) at
// or above it, by one wave (MSB-first 8-bit digits; digits on which all
// keys agree cost nothing).
__device__ __forceinline__ uint64_t wave_kth(const uint64_t* wb, uint32_t n, uint32_t rank, uint32_t* hist) {
  const uint32_t lane = threadIdx.x & 63u;
  wave_lds_sync();  // the list was just written by other lanes
  uint64_t a_and = ~0ull, a_or = 0ull;
  for (uint32_t i = lane; i < n; i += 64) {
    const uint64_t K = wb[i];
    a_and &= K;
    a_or |= K;
  }
  a_and = wave_and_u64(a_and);
  a_or = wave_or_u64(a_or);
  const uint64_t varies = a_and ^ a_or;
  uint64_t prefix = 0;
  uint32_t rem = rank;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (((varies >> shift) & 0xFFull) == 0) {
      prefix |= a_and & (0xFFull << shift);
      continue;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0u;
    wave_lds_sync();
    const uint64_t hmask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
    for (uint32_t i = lane; i < n; i += 64) {
      const uint64_t K = wb[i];
      if ((K & hmask) == prefix) atomicAdd(&hist[(uint32_t)(K >> shift) & 255u], 1u);
    }
    wave_lds_sync();
    uint32_t c[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) c[b] = hist[255 - 4 * lane - b];
    wave_lds_sync();
    const uint32_t local = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan_u32(local, (int)lane);
    uint32_t cum = incl - local;
    const bool mine = cum < rem && rem <= incl;
    uint32_t d = 0, r2 = 0, bc = 0;
    if (mine) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (cum + c[b] >= rem) {
          d = 255 - 4 * lane - b;
          r2 = rem - cum;
          bc = c[b];
          break;
        }
        cum += c[b];
      }
    }
    const int src = __builtin_ctzll(__ballot(mine));  // exactly one lane
    d = (uint32_t)__builtin_amdgcn_readlane((int)d, src);
    r2 = (uint32_t)__builtin_amdgcn_readlane((int)r2, src);
    bc = (uint32_t)__builtin_amdgcn_readlane((int)bc, src);
    prefix |= (uint64_t)d << shift;
    rem = r2;
    if (bc == rem) break;  // the whole bucket qualifies
  }
  return prefix;
}

// Keep the keys of wb[0..n) at or above T, in place (a key's destination
// never lies past the chunk being read); returns their number.
__device__ __forceinline__ uint32_t wave_cut(uint64_t* wb, uint32_t n, uint64_t T) {
  const uint32_t lane = threadIdx.x & 63u;
  wave_lds_sync();
  uint32_t base = 0;
  for (uint32_t c0 = 0; c0 < n; c0 += 64) {
    const uint32_t i = c0 + lane;
    const uint64_t K = i < n ? wb[i] : 0ull;
    const bool keep = i < n && K >= T;
    const uint64_t m = __ballot(keep);
    wave_lds_sync();
    if (keep) wb[base + lane_rank(m)] = K;
    base += (uint32_t)__popcll(m);
  }
  wave_lds_sync();
  return base;
}

// LDS use (about 33 KB) allows four workgroups per CU, i.e. four waves per
// SIMD; the attribute lets the compiler use the 128 VGPRs that occupancy
// leaves instead of spilling to reach a higher one.
template <typename DT, bool WANT_LSE, bool MOM = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 4))) void topk_wave_kernel(TopkArgs a) {
  constexpr int E = Elem<DT>::E;
  constexpr int64_t TILE = (int64_t)NT * WTG * E;
  constexpr uint32_t kBlockCap = NWAVE * kWCap;  // the lists, then the row's merge buffer
  __shared__ __attribute__((aligned(16))) uint64_t s_key[kBlockCap];
  __shared__ WaveArea area_all[NWAVE];
  __shared__ uint32_t wcount[NWAVE];
  // Shared threshold.  Wave w publishes in s_slot[w] a key with at least
  // ceil(k/4) of its own elements at or above it; the four waves' elements
  // are distinct, so at least k elements reach the smallest slot, which
  // makes min(s_slot) (and s_T, the largest such minimum seen) a valid
  // lower bound of the segment's k-th largest key for every wave.
  __shared__ uint64_t s_slot[NWAVE];
  __shared__ uint64_t s_T;
  // Histogram of lane maxima (one per lane and tile, so distinct
  // elements) that reach the threshold: bin b counts maxima whose value key
  // is at least hbase + (b << 16) (the last bin: and above).  The lower edge
  // of the highest bin at which the count from the top reaches k is a valid
  // threshold for every wave.
  __shared__ uint32_t s_hist[256];
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
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  const uint32_t e_full32 = (uint32_t)e_full;
  const float c = kLog2e;
  const uint32_t select_at = min(max(2u * k, 192u), kWCap - 64u);

  if (tid == 0) s_T = 1;  // ordered before every read by the first barrier below
  if (lane == 0) s_slot[wave] = 1;  // each wave its own slot, before it publishes
  s_hist[tid] = 0u;                   // ordered before use by the first barrier below
  uint32_t hbase = 0;                 // value key of the first threshold
  WaveArea& area = area_all[wave];
  uint64_t* wb = s_key + wave * kWCap;
  uint32_t wcnt = 0;  // records in this wave's list
  uint32_t sn = 0;    // staged groups (may pass kWStage: the tile then overflows)
  uint64_t T = 1;     // every real element's composite key is above 1
  float tf = -__builtin_inff();

  // Lane log-sum-exp with a lazy offset om (in input units): LS is the
  // lane's sum of 2^((x - om) c) in float64.  Terms are exp2(fma(x, c, noff))
  // with noff = -fl(om c); these carry the factor 2^delta of that rounding,
  // delta = om c - fl(om c), which corr = 2^-delta removes when a tile is
  // folded in.  Past |om| = 2^25 the rounding could reach the exponent
  // range, and the lane takes its terms exactly as exp2((x - om) c) instead
  // (huge).  trig: a tile maximum above it moves the offset.
  float lm = -__builtin_inff(), om = -__builtin_inff(), trig = -__builtin_inff(), noff = 0.0f, ls = 0.0f;
  double LS = 0.0, corr = 1.0;
  bool huge = false;
  // Move the offset to m (finite, above the current one), rescaling LS.
  auto set_offset = [&](float m) {
    LS = (om == -__builtin_inff()) ? 0.0 : LS * exp2_split(((double)om - (double)m) * (double)c);
    om = m;
    const float oc = m * c;
    noff = -oc;
    trig = m + kLazyLog2 / c;
    corr = exp2_split((double)oc - (double)m * (double)c);
    huge = !(__builtin_fabsf(m) <= 0x1p25f);
  };

  // Row moments for top-n-sigma (MOM): each lane's values above -inf, shifted
  // by its first such value, in float64 (as the moments pass takes them).
  // The shift is settled once per group, in the rare groups a lane meets
  // before its first such value, and the count is an integer, so an element
  // costs a conversion, a subtraction, a select, an add and an FMA.
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

  auto group_max = [&](const Group& g, float (&x)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = __uint_as_float(gbits<DT>(g, e));
    float m0 = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) m0 = fmax_nan(m0, x[e]);
    return m0;
  };

  auto stage = [&](const Group& g, float gm, uint32_t e0) {
    const bool pass = gm >= tf;
    const uint64_t bm = __ballot(pass);
    if (bm) {
      const uint32_t p = sn + lane_rank(bm);
      if (pass && p < kWStage) {
#pragma unroll
        for (int i = 0; i < 4; ++i) area.w[p][i] = g.w[i];
        area.e0[p] = e0;
      }
      sn += (uint32_t)__popcll(bm);
    }
  };

  // The histogram's threshold, published in s_T (one wave a tile does
  // this): lane l reads bins 255-4l .. 252-4l, a wave prefix sum counts
  // from the top.
  auto hist_threshold = [&]() {
    uint32_t c4[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) c4[b] = __hip_atomic_load(&s_hist[255 - 4 * lane - b], __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t local = c4[0] + c4[1] + c4[2] + c4[3];
    const uint32_t incl = wave_incl_scan_u32(local, lane);
    uint32_t cum = incl - local;
    const bool mine = cum < k && k <= incl;
    uint32_t bin = 0;
    if (mine) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (cum + c4[b] >= k) {
          bin = 255 - 4 * lane - b;
          break;
        }
        cum += c4[b];
      }
    }
    const uint64_t who = __ballot(mine);
    if (who) {
      bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, __builtin_ctzll(who));
      const uint64_t Th = (uint64_t)(hbase + (bin << 16)) << 32;
      if (lane == 0) atomicMax(reinterpret_cast<unsigned long long*>(&s_T), (unsigned long long)Th);
    }
  };

  // Add a lane maximum (a real element, seen for the first time) that
  // reaches the threshold to the histogram.
  auto count_max = [&](float m) {
    const uint32_t hk = fkey(__float_as_uint(m));
    if (m >= tf && hk >= hbase) atomicAdd(&s_hist[min(255u, (hk - hbase) >> 16)], 1u);
  };

  // Maximum and log-sum-exp terms of one group against the lane's current
  // offset (no branch); returns the group maximum.
  auto lse_group = [&](const Group& g) {
    float x[E];
    const float gm = group_max(g, x);
    mom_add(x);
    if constexpr (WANT_LSE) {
      float acc = __builtin_amdgcn_exp2f(fmaf(x[0], c, noff));
#pragma unroll
      for (int e = 1; e < E; ++e) acc += __builtin_amdgcn_exp2f(fmaf(x[e], c, noff));
      ls += acc;
    }
    return gm;
  };

  // After a tile's terms are in ls: a lane whose tile maximum passed its
  // trigger moves its offset to that maximum; it, and a lane past the
  // fast-path range, recompute the tile's terms (the ones just added may
  // have overflowed).
  auto lse_check = [&](auto& g, float tmax) {
    lm = fmax_nan(lm, tmax);
    if constexpr (WANT_LSE) {
      constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
      const bool up = tmax > trig && tmax < __builtin_inff();
      if (__ballot(up || huge)) {
        if (up) set_offset(tmax);
        if (up || huge) {
          // fresh words (not the values unpacked above, which would then
          // stay live through the whole tile)
          auto fresh = [&](int j, float (&x)[E]) {
            uint32_t w0 = g[j].w[0], w1 = g[j].w[1], w2 = g[j].w[2], w3 = g[j].w[3];
            asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
            Group gf;
            gf.w[0] = w0; gf.w[1] = w1; gf.w[2] = w2; gf.w[3] = w3;
            (void)group_max(gf, x);
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

  // Make room in the wave's list: publish the wave's ceil(k/4)-th largest
  // key, take the shared threshold, drop what falls below it, and only if
  // the list is still long cut it to the wave's own k largest.
  auto shrink = [&]() {
    const uint32_t q = (k + NWAVE - 1) / NWAVE;
    if (wcnt > q) {
      const uint64_t Tq = wave_kth(wb, wcnt, q, area.hist);
      if (lane == 0) {
        const uint64_t mine = max(Tq, __hip_atomic_load(&s_slot[wave], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        __hip_atomic_store(&s_slot[wave], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        uint64_t mn = mine;
#pragma unroll
        for (int q2 = 0; q2 < NWAVE; ++q2)
          mn = min(mn, __hip_atomic_load(&s_slot[q2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        atomicMax(reinterpret_cast<unsigned long long*>(&s_T), (unsigned long long)mn);
      }
      wave_lds_sync();
    }
    const uint64_t Ts = uniform_u64(__hip_atomic_load(&s_T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (Ts > T) T = Ts;
    wcnt = wave_cut(wb, wcnt, T);
    if (wcnt > select_at) {
      T = wave_kth(wb, wcnt, k, area.hist);
      wcnt = wave_cut(wb, wcnt, T);
    }
    tf = thr_float(T);
  };

  // Append every element of the staged groups that reaches T to the wave's
  // list.  Each lane opens one staged group per step (64 groups a step) and
  // a wave prefix sum of the lanes' counts places the appends.  A step that
  // would overflow the list goes element by element instead (at most 64
  // appends each), shrinking the list whenever one would not fit: shrink
  // leaves at most select_at <= kWCap - 64 records, so every such append
  // fits and the flush always progresses.  (One call site of shrink only:
  // a second inlined copy makes the compiler put locals in scratch.)
  auto flush = [&]() {
    wave_lds_sync();
    for (uint32_t q0 = 0; q0 < sn; q0 += 64) {
      const uint32_t q = q0 + (uint32_t)lane;
      const bool has = q < sn;
      Group gg;
      uint32_t e0 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) gg.w[i] = has ? area.w[q][i] : 0u;
      if (has) e0 = area.e0[q];
      uint32_t pm = 0;  // this lane's elements that reach T
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t id = e0 + (uint32_t)e;
        const bool pass = has && id < e_full32 && comp_key(gbits<DT>(gg, e), id) >= T;
        pm |= pass ? (1u << e) : 0u;
      }
      const uint32_t cnt = (uint32_t)__popc(pm);
      const uint32_t incl = wave_incl_scan_u32(cnt, lane);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (wcnt + total <= kWCap) {
        uint32_t pos = wcnt + incl - cnt;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (pm & (1u << e)) wb[pos++] = comp_key(gbits<DT>(gg, e), e0 + (uint32_t)e);
        wcnt += total;
      } else {
        for (int e = 0; e < E; ++e) {
          // element e without indexing the group by a runtime value (that
          // would put it in scratch memory): select the word, then the half
          const int wi = (E == 8) ? (e >> 1) : e;
          const uint32_t wd = wi == 0 ? gg.w[0] : wi == 1 ? gg.w[1] : wi == 2 ? gg.w[2] : gg.w[3];
          const uint32_t b = (E == 8) ? ((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16)) : wd;
          const uint64_t K = comp_key(b, e0 + (uint32_t)e);
          bool pass = ((pm >> e) & 1u) && K >= T;
          uint64_t m = __ballot(pass);
          if (wcnt + (uint32_t)__popcll(m) > kWCap) {
            shrink();
            pass = pass && K >= T;
            m = __ballot(pass);
          }
          if (pass) wb[wcnt + lane_rank(m)] = K;
          wcnt += (uint32_t)__popcll(m);
        }
      }
    }
    sn = 0;
    wave_lds_sync();
    tf = thr_float(T);
  };

  // First tile: threshold from the lane maxima m (needs k <= 4 waves x 64),
  // and the lane's first exp2 offset.
  auto first_threshold = [&](float m, int64_t t0) {
    if constexpr (WANT_LSE) {
      if (m > -__builtin_inff() && m < __builtin_inff()) set_offset(m);
    }
    const bool real = t0 + (int64_t)tid * E < e_full;
    const uint32_t lk = real ? fkey(__float_as_uint(m)) : 0u;
    const uint32_t kw = (k + NWAVE - 1) / NWAVE;
    uint32_t tw = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = tw | (1u << b);
      if ((uint32_t)__popcll(__ballot(lk >= cand)) >= kw) tw = cand;
    }
    if (lane == 0) {
      sh.wtau[wave] = tw;
      s_slot[wave] = (uint64_t)tw << 32;  // this wave has ceil(k/4) elements there
    }
    __syncthreads();
    uint32_t tau = sh.wtau[0];
#pragma unroll
    for (int q = 1; q < NWAVE; ++q) tau = min(tau, sh.wtau[q]);
    const uint64_t Tn = (uint64_t)tau << 32;
    if (Tn > T) T = Tn;
    hbase = tau;
    if (tid == 0) atomicMax(reinterpret_cast<unsigned long long*>(&s_T), (unsigned long long)Tn);
    tf = thr_float(T);
  };
  // Lane maximum of a tile, for the first threshold; the asm keeps the
  // compiler from sharing these unpacked values with the pass that follows.
  auto first_tile = [&](auto& g, int64_t t0) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NGP; ++j) {
      float x[E];
      m = fmax_nan(m, group_max(g[j], x));
    }
#pragma unroll
    for (int j = 0; j < NGP; ++j) asm volatile("" : "+v"(g[j].w[0]), "+v"(g[j].w[1]), "+v"(g[j].w[2]), "+v"(g[j].w[3]));
    first_threshold(m, t0);
  };

  // Streaming loop.  Every flush happens at the top of the loop, so the
  // flush (and the select inside it) is one piece of code and no tile data
  // is live across it.  A tile whose passing groups did not fit the staging
  // list is taken again from memory, one group per lane at a time, after
  // the groups staged before it are opened (its log-sum-exp terms are
  // already in).
  const int64_t e_tiles = e_begin + (e_full - e_begin) / TILE * TILE;
  // Fair progress: the SIMD arbiter favours older waves, so without help
  // the first of the workgroups sharing a CU races ahead and the last one
  // ends alone, too few waves in flight to keep HBM busy.  A wave starts at
  // the highest issue priority and drops one level per quarter of its
  // tiles, so waves that are ahead yield to those behind; the quarters of a
  // younger workgroup end one tile later per step of age.  (Workgroups are
  // dealt to the CUs in turn, so in a grid of four per CU the age rank is
  // blockIdx * 4 / gridDim; in other grids the shift is merely harmless.)
  const uint32_t ntiles = (uint32_t)((e_tiles - e_begin) / TILE);
  const uint32_t age = (blockIdx.x * 4u) / gridDim.x;
  const uint32_t q1 = ntiles / 4 + age, q2 = ntiles / 2 + age, q3 = ntiles - ntiles / 4 + age;
  __builtin_amdgcn_s_setprio(3);
  int64_t t0 = e_begin;
  int64_t ov_t0 = 0;
  uint32_t ov_lim = 0;  // elements of the overflowed tile inside the segment (a multiple of E)
  int ovj = WTG;        // next group of an overflowed tile to take again (WTG: none)
  bool first = true, want_flush = false;
  uint32_t tix = 0;  // full tiles so far (the histogram scan rotates over the waves)
  for (;;) {
    if (want_flush) {
      flush();
      want_flush = false;
    }
    if (ovj < WTG) {
      const uint32_t o = (uint32_t)(ovj * NT + tid) * E;
      Group g1;
      if constexpr (!WANT_LSE && !MOM) {
        // (a partial tile can overflow in this variant: its groups past the
        // segment's end read as -inf and are not loaded, and ovj stops at
        // the first group no lane reaches)
        const bool full = o < ov_lim;
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + ov_t0 + (full ? o : 0u)));
        constexpr uint32_t pad = (E == 4) ? kNegInfBits : 0xFF80FF80u;
        g1.w[0] = full ? v.x : pad;
        g1.w[1] = full ? v.y : pad;
        g1.w[2] = full ? v.z : pad;
        g1.w[3] = full ? v.w : pad;
      } else {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + ov_t0 + o));
        g1.w[0] = v.x; g1.w[1] = v.y; g1.w[2] = v.z; g1.w[3] = v.w;
      }
      float x[E];
      stage(g1, group_max(g1, x), (uint32_t)ov_t0 + o);
      ++ovj;
      if constexpr (!WANT_LSE && !MOM)
        if ((uint32_t)(ovj * NT) * E >= ov_lim) ovj = WTG;
      want_flush = true;
      continue;
    }
    if (t0 < e_tiles) {
      Group g[WTG];
      load_tile_buf<DT, WTG>(g, xr + t0);
      if (first) {
        first_tile(g, t0);
        first = false;
      }
      // the shared threshold, read early (used after the exp2 work)
      const uint64_t Ts = uniform_u64(__hip_atomic_load(&s_T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      const uint32_t sn0 = sn;
      float gm[WTG];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < WTG; ++j) {
        gm[j] = lse_group(g[j]);
        tmax = fmax_nan(tmax, gm[j]);
      }
      // finish the exp2 terms before the branches below (otherwise the
      // compiler keeps many groups unpacked at once)
      if constexpr (WANT_LSE) asm volatile("" ::"v"(ls), "v"(tmax));
      lse_check(g, tmax);
      if (Ts > T) {
        T = Ts;
        tf = thr_float(T);
      }
#pragma unroll
      for (int j = 0; j < WTG; ++j) stage(g[j], gm[j], (uint32_t)t0 + (uint32_t)(j * NT + tid) * E);
      count_max(tmax);
      fold();
      if ((tix++ & (NWAVE - 1)) == (uint32_t)wave) hist_threshold();
      if (tix == q1) __builtin_amdgcn_s_setprio(2);
      else if (tix == q2) __builtin_amdgcn_s_setprio(1);
      else if (tix == q3) __builtin_amdgcn_s_setprio(0);
      if (sn > kWStage) {
        sn = sn0;  // open the earlier groups, then take this tile again
        ov_t0 = t0;
        if constexpr (!WANT_LSE && !MOM) ov_lim = (uint32_t)TILE;
        ovj = 0;
        want_flush = true;
      } else if (sn >= kFlushAt) {
        want_flush = true;
      }
      t0 += TILE;
      continue;
    }
    if (t0 < e_full) {
      if constexpr (!WANT_LSE && !MOM) {
        // the segment's last partial tile in one memory round trip instead
        // of one per group: all its loads issued together (groups past
        // e_full read as -inf), then the same steps as a full tile on the
        // ngr groups that hold real elements only
        const uint32_t lim = (uint32_t)(e_full - t0);
        const uint32_t ngr = (lim + (uint32_t)(NT * E) - 1u) / (uint32_t)(NT * E);  // uniform, 1..WTG
        Group g[WTG];
        load_tile_buf_part<DT, WTG>(g, xr + t0, lim);
        if (first) {
          first_tile(g, t0);
          first = false;
        }
        const uint64_t Ts = uniform_u64(__hip_atomic_load(&s_T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        const uint32_t sn0 = sn;
        float gm[WTG];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < WTG; ++j) {
          gm[j] = -__builtin_inff();
          if ((uint32_t)j < ngr) {
            gm[j] = lse_group(g[j]);
            tmax = fmax_nan(tmax, gm[j]);
          }
        }
        lse_check(g, tmax);
        if (Ts > T) {
          T = Ts;
          tf = thr_float(T);
        }
#pragma unroll
        for (int j = 0; j < WTG; ++j)
          if ((uint32_t)j < ngr) stage(g[j], gm[j], (uint32_t)t0 + (uint32_t)(j * NT + tid) * E);
        if ((uint32_t)tid * E < lim) count_max(tmax);  // lanes holding a real group
        fold();
        if (sn > kWStage) {
          sn = sn0;  // open the earlier groups, then take this tile again
          ov_t0 = t0;
          ov_lim = lim;
          ovj = 0;
          want_flush = true;
        } else if (sn >= kFlushAt) {
          want_flush = true;
        }
        t0 = e_full;
        continue;
      } else {
        // the row's last partial tile, one group per lane at a time: with
        // float work on every element, the tile at once measured slower (at
        // most 63 staged groups wait, so these never overflow the staging
        // list)
        Group g1[1];
        load_tile<DT, 1, true>(g1, xr, t0, e_full);
        if (first) {
          first_tile(g1, t0);
          first = false;
        }
        const float gm1 = lse_group(g1[0]);
        lse_check(g1, gm1);
        stage(g1[0], gm1, (uint32_t)t0 + (uint32_t)tid * E);
        if (t0 + (int64_t)tid * E < e_full) count_max(gm1);  // real groups only
        fold();
        if (sn >= kFlushAt) want_flush = true;
        t0 += (int64_t)NT * E;
        continue;
      }
    }
    if (sn) {
      want_flush = true;
      continue;
    }
    break;
  }

  // The row's last few elements (fewer than one group): lanes of wave 0.
  if (e_full < e_end && wave == 0) {
    const int64_t i = e_full + lane;
    const bool has = i < e_end;
    const uint32_t b = has ? gbits_at<DT>(xr, i) : kNegInfBits;
    const float x = __uint_as_float(b);
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
    // room for the (at most E - 1) keys: a flush may have left the list full,
    // so cut it first then, to the shared threshold and if need be to the
    // wave's own k largest (k <= kWCap - 8)
    if (wcnt > kWCap - 8u) {
      const uint64_t Ts = uniform_u64(__hip_atomic_load(&s_T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      if (Ts > T) T = Ts;
      wcnt = wave_cut(wb, wcnt, T);
      if (wcnt > kWCap - 8u) {
        T = wave_kth(wb, wcnt, k, area.hist);
        wcnt = wave_cut(wb, wcnt, T);
      }
    }
    const uint64_t K = comp_key(b, (uint32_t)i);
    const bool pass = has && K >= T;
    const uint64_t m = __ballot(pass);
    if (pass) wb[wcnt + lane_rank(m)] = K;
    wcnt += (uint32_t)__popcll(m);
  }
  // End of the segment, in four barriers.
  // (1) Each wave's log-sum-exp (relative to the wave's maximum) and its
  //     threshold go to LDS.
  LSE r{lm, 0.0};
  if constexpr (WANT_LSE) {
    if (lm != lm || lm == __builtin_inff()) r.s = __builtin_nan("");
    else if (lm != -__builtin_inff()) r.s = LS * exp2_split(((double)om - (double)lm) * (double)c);
  }
  {
    const float Mw = wave_max_nan(r.m);
    double t = 0.0;
    if (Mw != Mw || Mw == __builtin_inff()) t = __builtin_nan("");
    else if (r.m != -__builtin_inff()) t = r.s * exp2_split(((double)r.m - (double)Mw) * (double)c);
    t = wave_sum_f64(t);
    if (lane == 0) {
      sh.wm[wave] = Mw;
      sh.ws[wave] = t;
      atomicMax(reinterpret_cast<unsigned long long*>(&s_T), (unsigned long long)T);
    }
  }
  __syncthreads();
  // (2) The workgroup's log-sum-exp (every thread), and each wave's records
  //     that reach the final shared threshold (at least k in all: it is some
  //     wave's k-th largest, a valid histogram bound, or the first tile's
  //     bound), taken into registers with their place among the wave's kept.
  {
    float M = sh.wm[0];
#pragma unroll
    for (int q = 1; q < NWAVE; ++q) M = fmax_nan(M, sh.wm[q]);
    double S = 0.0;
    if (M != M || M == __builtin_inff()) {
      S = __builtin_nan("");
    } else {
#pragma unroll
      for (int q = 0; q < NWAVE; ++q)
        if (sh.wm[q] != -__builtin_inff()) S += sh.ws[q] * exp2_split(((double)sh.wm[q] - (double)M) * (double)c);
    }
    r = LSE{M, S};
  }
  constexpr uint32_t kPer = kWCap / 64;
  uint64_t held[kPer];
  uint32_t place[kPer];
  {
    uint64_t Tb = s_T > T ? s_T : T;
    // When the four lists can each be cut to their k largest and still fit the
    // direct ranking (4 k <= kRank), a wave holding more than k records above
    // the shared threshold cuts to its own k largest (a wave-level select, no
    // barrier): the workgroup's k largest lie among the waves' k largest, and
    // the radix select of more than kRank records is avoided.
    if (4u * k <= kRank) {
      uint32_t above = 0;
#pragma unroll
      for (uint32_t q = 0; q < kPer; ++q) {
        const uint32_t i = q * 64 + lane;
        above += (uint32_t)__popcll(__ballot(i < wcnt && wb[i] >= Tb));
      }
      if (above > k) {
        const uint64_t Tw = wave_kth(wb, wcnt, k, area.hist);
        Tb = Tw > Tb ? Tw : Tb;
      }
    }
    uint32_t kept = 0;
#pragma unroll
    for (uint32_t q = 0; q < kPer; ++q) {
      const uint32_t i = q * 64 + lane;
      held[q] = wb[i];  // i < kWCap: inside the wave's list; entries past wcnt are masked
      const bool keep = i < wcnt && held[q] >= Tb;
      const uint64_t m = __ballot(keep);
      place[q] = keep ? kept + lane_rank(m) : 0xFFFFFFFFu;
      kept += (uint32_t)__popcll(m);
    }
    wcnt = kept;
  }
  if (lane == 0) wcount[wave] = wcnt;
  __syncthreads();
  // (3) Every wave writes its kept records to their place at the front of
  //     s_key (the lists are all in registers by now), then zeros after them.
  uint32_t off = 0, n = 0;
#pragma unroll
  for (int q = 0; q < NWAVE; ++q) {
    if (q < wave) off += wcount[q];
    n += wcount[q];
  }
#pragma unroll
  for (uint32_t q = 0; q < kPer; ++q)
    if (place[q] != 0xFFFFFFFFu) s_key[off + place[q]] = held[q];
  if (n <= kRank && tid < 8) s_key[n + tid] = 0ull;  // (else the select below pads)
  __syncthreads();
  // (4) Winners in (value desc, id asc) order at okey: more than kRank
  //     records are first cut to k by the radix select; then each record's
  //     rank among the rest is its place (ranks >= k drop out).
  uint64_t* okey = s_key + kBlockCap / 2;
  auto rank_order = [&](uint32_t& nn, bool padded) {
    if (nn > kRank) {
      select_compact<kBlockCap>(sh, s_key, nullptr, nn, k);
      nn = k;
      padded = false;
    }
    if (!padded) {
      // zeros after the keys (never above a real key), so the count runs in
      // whole blocks of 8: two keys per 16-byte read, four reads in flight
      if (tid < 8) s_key[nn + tid] = 0ull;
      __syncthreads();
    }
    if ((uint32_t)tid < nn) {
      const uint64_t K = s_key[tid];
      uint32_t r0 = 0;
      const uint32_t n8 = (nn + 7u) & ~7u;
      for (uint32_t j = 0; j < n8; j += 8) {
        const u64x2 q0 = *reinterpret_cast<const u64x2*>(&s_key[j]);
        const u64x2 q1 = *reinterpret_cast<const u64x2*>(&s_key[j + 2]);
        const u64x2 q2 = *reinterpret_cast<const u64x2*>(&s_key[j + 4]);
        const u64x2 q3 = *reinterpret_cast<const u64x2*>(&s_key[j + 6]);
        r0 += (uint32_t)(q0.x > K) + (uint32_t)(q0.y > K) + (uint32_t)(q1.x > K) + (uint32_t)(q1.y > K) +
              (uint32_t)(q2.x > K) + (uint32_t)(q2.y > K) + (uint32_t)(q3.x > K) + (uint32_t)(q3.y > K);
      }
      if (r0 < k) okey[r0] = K;
    }
    __syncthreads();
    nn = min(nn, k);
  };
  rank_order(n, n <= kRank);

  // Row moments (MOM): the lanes' sums folded per wave, then the waves in
  // order; then the segments (below), in a fixed order too.
  __shared__ double s_mom[3 * NWAVE];
  Mom mv{0.0, 0.0, 0.0};
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
  if constexpr (MOM) {
    const double mn = (double)mcnt;
    Mom v{mn, 0.0, 0.0};
    if (mn > 0.0) v = Mom{mn, mr + ms1 / mn, ms2 - ms1 * ms1 / mn};
    mv = fold_waves(v);
  }

  if (a.S > 1) {
    const int64_t slot = row * a.S + seg;
    for (uint32_t i = tid; i < n; i += NT) st_dev(&a.rec_key[slot * k + i], okey[i]);
    if (tid == 0) {
      st_dev(&a.rec_cnt[slot], n);
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
    // one round of loads: the segments' counts, their (max, sum) partials and
    // every record slot (a segment's slots past its count hold stale keys,
    // dropped below); threads past the segments load segment 0's words and
    // drop them, so no load waits on a branch
    const int64_t s_t = s0 + (tid < a.S ? tid : 0);
    const uint32_t cnt_l = ld_dev(&a.rec_cnt[s_t]);
    constexpr int kSlotQ = kCapSmall / NT;
    const uint32_t nslots = (uint32_t)a.S * k;  // <= kCapSmall (the segment plan)
    uint64_t v[kSlotQ];
#pragma unroll
    for (int q = 0; q < kSlotQ; ++q) {
      const uint32_t f = (uint32_t)(q * NT) + tid;
      if (f < nslots) v[q] = ld_dev(&a.rec_key[s0 * k + f]);
    }
    // this thread's segment's moments (MOM; masked where they are used, so
    // that nothing waits for them before)
    Mom ms{0.0, 0.0, 0.0};
    if constexpr (MOM) ms = Mom{ld_dev(&a.m_n[s_t]), ld_dev(&a.m_mean[s_t]), ld_dev(&a.m_m2[s_t])};
    const uint32_t cnt_t = tid < a.S ? cnt_l : 0u;
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
    // slot (segment sg, index i) -> the concatenation, if i is below sg's count
#pragma unroll
    for (int q = 0; q < kSlotQ; ++q) {
      const uint32_t f = (uint32_t)(q * NT) + tid;
      if (f < nslots) {
        const uint32_t sg = f / k, i = f - sg * k;
        const uint32_t o = sh.hist[sg], e = (int)sg + 1 < a.S ? sh.hist[sg + 1] : n;
        if (o + i < e) s_key[o + i] = v[q];
      }
    }
    __syncthreads();
    rank_order(n, false);
    if constexpr (MOM) mv = fold_waves(tid < a.S ? ms : Mom{0.0, 0.0, 0.0});
  }
  double sigma = a.sigma ? a.sigma[row] : 0.0;
  if constexpr (MOM) sigma = mv.n > 0.0 ? sqrt(fmax(mv.m2, 0.0) / mv.n) : 0.0;

  const bool bad = (r.m != r.m) || (r.m == __builtin_inff());
  const bool none = bad || r.m == -__builtin_inff();
  // A winner's bits from its key; +-0 (one key) from the row itself.
  auto win_bits = [&](uint64_t K) -> uint32_t {
    const uint32_t hk = (uint32_t)(K >> 32);
    return (hk == 0x80000000u) ? gbits_at<DT>(xr, (int64_t)(~(uint32_t)K)) : key_bits(hk);
  };
  if (a.mode == 0) {
    for (uint32_t j = tid; j < k; j += NT) {
      const bool ok = !bad && j < n;
      const uint64_t K = ok ? okey[j] : 0ull;
      a.out_ids[row * k + j] = ok ? ~(uint32_t)K : kFail;
      a.out_vals[row * k + j] = ok ? __uint_as_float(win_bits(K)) : __builtin_nanf("");
    }
    if (tid == NT - 1) {  // a thread the loop above leaves idle (k <= 128)
      if (a.out_argmax) a.out_argmax[row] = (none || n == 0) ? kFail : ~(uint32_t)okey[0];
      if (a.out_lse)
        a.out_lse[row] = bad ? __builtin_nanf("")
                             : (r.m == -__builtin_inff() ? -__builtin_inff() : (float)((double)r.m + log(r.s)));
    }
  } else {
    uint32_t* obits = area_all[0].e0;  // free now; n <= k <= kWStage
    if (!none)
      for (uint32_t j = tid; j < n; j += NT) obits[j] = win_bits(okey[j]);
    __syncthreads();
    // the sampler chain; scratch in the lists' part of s_key and in a
    // staging area (free now)
    uint32_t tok = kFail;
    float lp = __builtin_nanf("");
    if (!none && n > 0) {
      double* E = reinterpret_cast<double*>(s_key);
      double* Sc = E + kWStage;
      uint32_t* ORD = &area_all[1].w[0][0];
      uint32_t* LIST = ORD + kWStage;
      const ChainParams cp{a.temperature, a.top_p,  a.top_n_sigma, a.typical_p, a.min_p,
                           a.mode == 2 ? a.out_kfl + row : nullptr, a.mode == 2 ? a.out_lse_f + row : nullptr};
      chain_tail(okey, obits, n, cp, sigma, a.u ? a.u[row] : 0.0f, E, Sc, ORD, LIST, &tok,
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

template <typename DT, bool L, bool M = false>
static hipError_t go_wave(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((topk_wave_kernel<DT, L, M>), dim3((unsigned)(a.rows * a.S)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_wave(int dtype, bool want_lse, const TopkArgs& a, hipStream_t s) {
  if (a.m_n)  // row moments in the same pass (the sampler chain's top-n-sigma; no log-sum-exp)
    return dtype == 0 ? go_wave<float, false, true>(a, s) : go_wave<uint16_t, false, true>(a, s);
  if (dtype == 0) return want_lse ? go_wave<float, true>(a, s) : go_wave<float, false>(a, s);
  return want_lse ? go_wave<uint16_t, true>(a, s) : go_wave<uint16_t, false>(a, s);
}

template <typename DT, bool L>
static int occ_wave() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, topk_wave_kernel<DT, L>, NT, 0) != hipSuccess) return 0;
  return n;
}

int topk_wave_blocks_per_cu(int dtype, bool want_lse) {
  if (dtype == 0) return want_lse ? occ_wave<float, true>() : occ_wave<float, false>();
  return want_lse ? occ_wave<uint16_t, true>() : occ_wave<uint16_t, false>();
}

}  // namespace vsel
