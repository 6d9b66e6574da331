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

constexpr int SG = 8;  // 16-byte groups per lane per tile

// One element of the log-sum-exp, for the few elements past the last whole
// group (one lane).
__device__ __forceinline__ void lse_push(LSE& st, float x, float c) {
  const float mn = fmax_nan(st.m, x);
  const float ms = (mn == -__builtin_inff()) ? 0.0f : mn;
  const double scale = (st.m == mn) ? 1.0 : (double)__builtin_amdgcn_exp2f((st.m - ms) * c);
  st.s = st.s * scale + (double)__builtin_amdgcn_exp2f((x - ms) * c);
  st.m = mn;
}

template <typename DT, bool WANT_LSE, bool VEC>
__global__ __launch_bounds__(NT) void scan_kernel(ScanArgs a) {
  constexpr int E = Elem<DT>::E;
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

  // Lane state: its first maximum (elements arrive in index order) and the
  // log-sum-exp pair.  A group is searched for its first maximum only when
  // its maximum beats the lane's best so far.
  float best = -__builtin_inff();
  uint32_t bidx = 0;
  LSE st{-__builtin_inff(), 0.0};
  auto tile = [&](const auto& g, int64_t t0) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
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
      if (m0 > best) {
        uint32_t f = E - 1;
#pragma unroll
        for (int e = E - 2; e >= 0; --e) f = (x[e] == m0) ? (uint32_t)e : f;
        best = m0;
        bidx = (uint32_t)t0 + (uint32_t)(j * NT + tid) * E + f;
      }
      if constexpr (WANT_LSE) {
        const float mn = fmax_nan(mt, m0);
        if (!(mn == mt)) {
          const float ms = (mn == -__builtin_inff()) ? 0.0f : mn;
          stile *= __builtin_amdgcn_exp2f((mt - ms) * c);
          ob = ms;
          mt = mn;
        }
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc += __builtin_amdgcn_exp2f((x[e] - ob) * c);
        stile += acc;
      } else {
        mt = fmax_nan(mt, m0);
      }
    }
    if constexpr (WANT_LSE) {
      // st.m < mt here unless equal; an empty state (st.m = -inf) scales to 0
      const double scale = (st.m == mt) ? 1.0 : (double)__builtin_amdgcn_exp2f((st.m - mt) * c);
      st.s = st.s * scale + (double)stile;
    }
    st.m = mt;
  };
  walk_groups<DT, SG, VEC>(xr, e_begin, e_full, tile);
  if (e_full < e_end && tid == 0) {
    for (int64_t i = e_full; i < e_end; ++i) {
      const float x = __uint_as_float(gbits_at<DT>(xr, i));
      if (x > best) {
        best = x;
        bidx = (uint32_t)i;
      }
      if constexpr (WANT_LSE) lse_push(st, x, c);
      else st.m = fmax_nan(st.m, x);
    }
  }

  uint64_t P = (best > -__builtin_inff()) ? (((uint64_t)fkey(__float_as_uint(best)) << 32) | (uint32_t)~bidx) : 0ull;
  P = wave_max_u64(P);
  LSE r = wave_lse(st, c);
  if (lane == 0) {
    sh.wk[wave] = P;
    sh.wm[wave] = r.m;
    sh.ws[wave] = r.s;
  }
  __syncthreads();
  P = sh.wk[0];
  r = LSE{sh.wm[0], sh.ws[0]};
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) {
    P = sh.wk[q] > P ? sh.wk[q] : P;
    r = lse_merge(r, LSE{sh.wm[q], sh.ws[q]}, c);
  }

  if (a.S > 1) {
    const int64_t slot = row * a.S + seg;
    if (tid == 0) {
      st_dev(&a.p_key[slot], P);
      st_dev(&a.p_m[slot], r.m);
      st_dev(&a.p_s[slot], r.s);
    }
    if (!last_done(sh, a.tickets + row, (uint32_t)a.S)) return;
    const int64_t s0 = row * a.S;
    merge_key_lse(sh, a.p_key + s0, a.p_m + s0, a.p_s + s0, a.S, c, P, r);
  }
  if (tid != 0) return;

  const bool bad = (r.m != r.m) || (r.m == __builtin_inff());
  const bool none = bad || P == 0;
  const uint32_t idx = none ? kFail : ~(uint32_t)P;
  if (a.out_idx) a.out_idx[row] = idx;
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
  if (a.vec1 && (a.rows2 == 0 || a.vec2))
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
