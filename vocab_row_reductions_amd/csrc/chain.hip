// chain.hip -- row moments for the top-n-sigma filter of the sampler chain
// ("Chapter 21", section 21.7: top_n_sigma masks the candidates against the
// maximum; the width is n standard deviations of the row's values).
//
// One pass over each row, one workgroup per (row, segment).  Each lane sums
// its values above -inf shifted by its own first such value (float64), so a
// row with a large common offset keeps its variance; lanes, waves and then
// segments merge their (count, mean, squared deviations) in a fixed order
// (the pairwise update of Chan, Golub and LeVeque), so the result is the
// same on every call.
#include "device.hpp"
#include "internal.hpp"

namespace vsel {


template <typename DT, bool VEC>
__global__ __launch_bounds__(NT) void moments_kernel(MomArgs a) {
  __shared__ SelShared sh;
  __shared__ double wn[NWAVE], wmean[NWAVE], wm2[NWAVE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Item it = work_item(a.S);
  const int64_t row = it.row;
  const int seg = (int)it.seg;
  if (row >= a.rows) return;
  const DT* __restrict__ xr = reinterpret_cast<const DT*>(a.x) + row * a.ld;
  const int64_t e_begin = (int64_t)seg * a.seg_len, e_end = min(a.V, e_begin + a.seg_len);
  // this thread's values, in the order the tiles give them; -inf (a mask)
  // takes no part (NaN rows fail closed elsewhere).  The shift r is settled
  // once per group, in the groups a lane meets before its first value above
  // -inf, and the count is an integer: per element a select, a conversion,
  // a subtraction, an add and an FMA.
  constexpr int E = Elem<DT>::E;
  uint32_t cnt = 0;
  double s1 = 0.0, s2 = 0.0, r = 0.0;
  auto add = [&](const float (&x)[E]) {
    if (cnt == 0u) {
      float first = -__builtin_inff();
#pragma unroll
      for (int e = E - 1; e >= 0; --e) first = x[e] > -__builtin_inff() ? x[e] : first;
      if (first > -__builtin_inff()) r = (double)first;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = x[e] > -__builtin_inff();
      const double d = ok ? (double)x[e] - r : 0.0;
      cnt += ok ? 1u : 0u;
      s1 += d;
      s2 = fma(d, d, s2);
    }
  };
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  walk_groups<DT, 4, VEC>(xr, e_begin, e_full, [&](const auto& g, int64_t) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
#pragma unroll
    for (int j = 0; j < NGP; ++j) {
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __uint_as_float(gbits<DT>(g[j], e));
      add(x);
    }
  });
  for (int64_t i = e_full + tid; i < e_end; i += NT) {  // the last few elements, one per lane
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = e == 0 ? __uint_as_float(gbits_at<DT>(xr, i)) : -__builtin_inff();
    add(x);
  }
  const double n = (double)cnt;
  Mom v{n, 0.0, 0.0};
  if (n > 0.0) v = Mom{n, r + s1 / n, s2 - s1 * s1 / n};
  v = wave_mom(v);
  if (lane == 0) {
    wn[wave] = v.n;
    wmean[wave] = v.mean;
    wm2[wave] = v.m2;
  }
  __syncthreads();
  if (tid == 0) {
    Mom w{0.0, 0.0, 0.0};
    for (int q = 0; q < NWAVE; ++q) w = mom_merge(w, Mom{wn[q], wmean[q], wm2[q]});
    v = w;
  }
  if (a.S > 1) {
    if (tid == 0) {
      st_dev(&a.p_n[row * a.S + seg], v.n);
      st_dev(&a.p_mean[row * a.S + seg], v.mean);
      st_dev(&a.p_m2[row * a.S + seg], v.m2);
    }
    if (!last_done(sh, a.tickets + row, (uint32_t)a.S)) return;
    // the segments' partials loaded at once (one per thread), then merged in
    // segment order by one thread
    __shared__ double pn[kMaxSegments], pmean[kMaxSegments], pm2[kMaxSegments];
    if (tid < a.S) {
      pn[tid] = ld_dev(&a.p_n[row * a.S + tid]);
      pmean[tid] = ld_dev(&a.p_mean[row * a.S + tid]);
      pm2[tid] = ld_dev(&a.p_m2[row * a.S + tid]);
    }
    __syncthreads();
    if (tid == 0) {
      Mom w{0.0, 0.0, 0.0};
      for (int sg = 0; sg < a.S; ++sg) w = mom_merge(w, Mom{pn[sg], pmean[sg], pm2[sg]});
      v = w;
    }
  }
  if (tid == 0) a.sigma[row] = v.n > 0.0 ? sqrt(fmax(v.m2, 0.0) / v.n) : 0.0;
}

hipError_t launch_moments(int dtype, const MomArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.S));
  if (dtype == 0) {
    if (a.vec)
      hipLaunchKernelGGL((moments_kernel<float, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((moments_kernel<float, false>), grid, dim3(NT), 0, s, a);
  } else {
    if (a.vec)
      hipLaunchKernelGGL((moments_kernel<uint16_t, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((moments_kernel<uint16_t, false>), grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vsel
