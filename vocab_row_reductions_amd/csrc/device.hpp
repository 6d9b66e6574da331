// device.hpp -- device building blocks shared by the vsel kernels (gfx950).
//
// Row layout: a workgroup of NT = 256 threads (4 wave64) walks a segment of
// one row in tiles.  A tile is G 16-byte groups per lane; lane l of the
// workgroup owns groups j*NT + l (j = 0..G-1) of the tile, so consecutive
// lanes load consecutive 16-byte words (fully coalesced) and every lane sees
// its own elements in increasing index order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsel {

constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
constexpr uint32_t kFail = 0xFFFFFFFFu;
constexpr uint32_t kNegInfBits = 0xFF800000u;
constexpr float kLog2e = 1.4426950408889634f;

// Elements per 16-byte group.
template <typename DT> struct Elem;
template <> struct Elem<float> { static constexpr int E = 4; };
template <> struct Elem<uint16_t> { static constexpr int E = 8; };  // bfloat16 bit patterns

struct Group { uint32_t w[4]; };
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float32 bit pattern of element e of a group (bfloat16 widens exactly).
template <typename DT> __device__ __forceinline__ uint32_t gbits(const Group& g, int e);
template <> __device__ __forceinline__ uint32_t gbits<float>(const Group& g, int e) { return g.w[e]; }
template <> __device__ __forceinline__ uint32_t gbits<uint16_t>(const Group& g, int e) {
  return (e & 1) ? (g.w[e >> 1] & 0xFFFF0000u) : (g.w[e >> 1] << 16);
}

// float32 bit pattern of element i of a row.
template <typename DT> __device__ __forceinline__ uint32_t gbits_at(const DT* row, int64_t i);
template <> __device__ __forceinline__ uint32_t gbits_at<float>(const float* row, int64_t i) { return __float_as_uint(row[i]); }
template <> __device__ __forceinline__ uint32_t gbits_at<uint16_t>(const uint16_t* row, int64_t i) { return (uint32_t)row[i] << 16; }

__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Load one full tile starting at tb (uniform): group j of this lane is
// elements (j*NT + threadIdx.x)*E .. +E-1.  Plain loads, issued back to back.
template <typename DT, int NG, bool VEC>
__device__ __forceinline__ void load_tile_full(Group (&g)[NG], const DT* __restrict__ tb) {
  constexpr int E = Elem<DT>::E;
  const uint32_t tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const uint32_t o = (uint32_t)(j * NT + tid) * E;
    if constexpr (VEC) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tb + o));
      g[j].w[0] = v.x; g[j].w[1] = v.y; g[j].w[2] = v.z; g[j].w[3] = v.w;
    } else if constexpr (E == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) g[j].w[e] = __float_as_uint(tb[o + e]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) g[j].w[q] = (uint32_t)tb[o + 2 * q] | ((uint32_t)tb[o + 2 * q + 1] << 16);
    }
  }
}

// Load one tile: group j of this lane covers elements
// t0 + (j*NT + threadIdx.x)*E .. +E-1, for whole groups below e_full (a
// multiple of E past e_begin); groups at or past e_full read as -inf.
// Addresses are a uniform tile base plus small 32-bit lane offsets, and all
// loads of the tile are issued back to back.  VEC rows (start and stride
// 16-byte aligned, e_begin a multiple of 8 elements) use 16-byte loads: an
// out-of-range group re-reads the tile's first group and is masked.  Other
// rows use element loads, clamped the same way.
template <typename DT, int NG, bool VEC>
__device__ __forceinline__ void load_tile(Group (&g)[NG], const DT* __restrict__ row, int64_t t0, int64_t e_full) {
  constexpr int E = Elem<DT>::E;
  constexpr uint32_t pad = (E == 4) ? kNegInfBits : 0xFF80FF80u;
  constexpr int64_t TILE = (int64_t)NT * NG * E;
  const uint32_t tid = threadIdx.x;
  const DT* __restrict__ tb = row + t0;                        // uniform
  const uint32_t lim = (uint32_t)min(e_full - t0, TILE);     // uniform, whole groups left (>= E)
  if (lim == (uint32_t)TILE) {                                 // full tile: plain loads
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const uint32_t o = (uint32_t)(j * NT + tid) * E;
      if constexpr (VEC) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tb + o));
        g[j].w[0] = v.x; g[j].w[1] = v.y; g[j].w[2] = v.z; g[j].w[3] = v.w;
      } else if constexpr (E == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) g[j].w[e] = __float_as_uint(tb[o + e]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) g[j].w[q] = (uint32_t)tb[o + 2 * q] | ((uint32_t)tb[o + 2 * q + 1] << 16);
      }
    }
    return;
  }
  // (the lane offsets of a partial tile are formed here, from a thread index
  // the compiler cannot hoist, so none of them stays live through a loop)
  uint32_t ptid = tid;
  asm volatile("" : "+v"(ptid));
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const uint32_t o = (uint32_t)(j * NT + ptid) * E;
    const bool full = o < lim;
    const uint32_t src = full ? o : 0u;
    if constexpr (VEC) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tb + src));
      g[j].w[0] = full ? v.x : pad;
      g[j].w[1] = full ? v.y : pad;
      g[j].w[2] = full ? v.z : pad;
      g[j].w[3] = full ? v.w : pad;
    } else if constexpr (E == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = __float_as_uint(tb[src + e]);
        g[j].w[e] = full ? v : pad;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t v = (uint32_t)tb[src + 2 * q] | ((uint32_t)tb[src + 2 * q + 1] << 16);
        g[j].w[q] = full ? v : pad;
      }
    }
  }
}

// Walk the whole groups of [e_begin, e_full) of a row: full tiles of NG
// groups per lane, then the remaining groups one per lane at a time (masked
// past e_full).  fn(g, t0) gets each tile (a Group[NG] or Group[1]) and its
// first element index; all threads call it for every tile.  The loads of the
// next full tile are in flight while fn works on the current one.
template <typename DT, int NG, bool VEC, class Fn>
__device__ __forceinline__ void walk_groups(const DT* __restrict__ xr, int64_t e_begin, int64_t e_full, Fn&& fn) {
  constexpr int E = Elem<DT>::E;
  constexpr int64_t TILE = (int64_t)NT * NG * E;
  const int64_t e_tiles = e_begin + (e_full - e_begin) / TILE * TILE;
  if (e_tiles > e_begin) {
    Group g[NG];
    load_tile_full<DT, NG, VEC>(g, xr + e_begin);
    for (int64_t t0 = e_begin; t0 < e_tiles; t0 += TILE) {
      Group n[NG];
      if (t0 + TILE < e_tiles) {
        load_tile_full<DT, NG, VEC>(n, xr + t0 + TILE);
      } else {
#pragma unroll
        for (int j = 0; j < NG; ++j) n[j] = g[j];
      }
      fn(g, t0);
#pragma unroll
      for (int j = 0; j < NG; ++j) g[j] = n[j];
    }
  }
  for (int64_t t0 = e_tiles; t0 < e_full; t0 += (int64_t)NT * E) {
    Group g1[1];
    load_tile<DT, 1, VEC>(g1, xr, t0, e_full);
    fn(g1, t0);
  }
}

// Every element of [e_begin, e_end) of a row: whole 16-byte groups through
// walk_groups (NG per lane per tile), then the last few elements one per
// lane.  fn(bits, i) gets the element's float32 bits and index; in a tile
// that ends early, padding elements (-inf, at indices past e_end) are passed
// too.  All threads call it the same number of times per tile.
template <typename DT, int NG, bool VEC, class Fn>
__device__ __forceinline__ void for_each_elem(const DT* __restrict__ xr, int64_t e_begin, int64_t e_end, Fn&& fn) {
  constexpr int E = Elem<DT>::E;
  const int64_t e_full = e_begin + (e_end - e_begin) / E * E;
  walk_groups<DT, NG, VEC>(xr, e_begin, e_full, [&](const auto& g, int64_t t0) {
    constexpr int NGP = (int)(sizeof(g) / sizeof(Group));
#pragma unroll
    for (int j = 0; j < NGP; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) fn(gbits<DT>(g[j], e), t0 + (int64_t)((j * NT + (int)threadIdx.x) * E + e));
  });
  for (int64_t i = e_full + threadIdx.x; i < e_end; i += NT) fn(gbits_at<DT>(xr, i), i);
}

// Order-preserving unsigned image of a float's bits: larger float -> larger
// key; -0.0 is folded onto +0.0 first so the two tie as floats do.
__device__ __forceinline__ uint32_t fkey(uint32_t u) {
  u = (u == 0x80000000u) ? 0u : u;
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_bits(uint32_t k) { return (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k; }

// Composite key: value first, then the lower id wins.  Distinct per element,
// and never 0 for a real element (its value key is >= the key of -inf).
__device__ __forceinline__ uint64_t comp_key(uint32_t bits, uint32_t id) {
  return ((uint64_t)fkey(bits) << 32) | (uint32_t)(~id);
}

// Float threshold for a composite threshold T: every element with composite
// >= T has value >= the returned float.
__device__ __forceinline__ float thr_float(uint64_t T) {
  uint32_t k = (uint32_t)(T >> 32);
  return (k <= 0x007FFFFFu) ? -__builtin_inff() : __uint_as_float(key_bits(k));
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((int)(uint32_t)v, m), hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  return __longlong_as_double((long long)shfl_xor_u64((uint64_t)__double_as_longlong(v), m));
}
// Wave all-reductions without LDS: four DPP steps inside each row of 16
// lanes (swap neighbours, swap pairs, mirror the half-row, mirror the row),
// after which every lane of a row holds the row's result; the four rows are
// combined through readlane.  Every lane of the wave must be active.
constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  return ((uint64_t)lane_u32((uint32_t)(v >> 32), l) << 32) | lane_u32((uint32_t)v, l);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<kDppXor1>(v));
  v = mx(v, dpp_u64<kDppXor2>(v));
  v = mx(v, dpp_u64<kDppHalfMirror>(v));
  v = mx(v, dpp_u64<kDppMirror>(v));
  return mx(mx(lane_u64(v, 0), lane_u64(v, 16)), mx(lane_u64(v, 32), lane_u64(v, 48)));
}
__device__ __forceinline__ float wave_max_nan(float v) {
  auto f = [](uint32_t u) { return __uint_as_float(u); };
  v = fmax_nan(v, f(dpp_u32<kDppXor1>(__float_as_uint(v))));
  v = fmax_nan(v, f(dpp_u32<kDppXor2>(__float_as_uint(v))));
  v = fmax_nan(v, f(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
  v = fmax_nan(v, f(dpp_u32<kDppMirror>(__float_as_uint(v))));
  const uint32_t u = __float_as_uint(v);
  return fmax_nan(fmax_nan(f(lane_u32(u, 0)), f(lane_u32(u, 16))), fmax_nan(f(lane_u32(u, 32)), f(lane_u32(u, 48))));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  auto d = [](uint64_t u) { return __longlong_as_double((long long)u); };
  auto u = [](double x) { return (uint64_t)__double_as_longlong(x); };
  v += d(dpp_u64<kDppXor1>(u(v)));
  v += d(dpp_u64<kDppXor2>(u(v)));
  v += d(dpp_u64<kDppHalfMirror>(u(v)));
  v += d(dpp_u64<kDppMirror>(u(v)));
  return (d(lane_u64(u(v), 0)) + d(lane_u64(u(v), 16))) + (d(lane_u64(u(v), 32)) + d(lane_u64(u(v), 48)));
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// ---------------------------------------------------------------- log-sum-exp
// (m, s): m is the running maximum (NaN-propagating, so a NaN or +inf element
// poisons it), s = sum exp2((x - m) * c) in float64 with c = log2(e)/T.
struct LSE { float m; double s; };

__device__ __forceinline__ LSE lse_merge(LSE a, LSE b, float c) {
  float M = fmax_nan(a.m, b.m);
  double sa = (a.m == M) ? a.s : a.s * exp2((double)(a.m - M) * (double)c);
  double sb = (b.m == M) ? b.s : b.s * exp2((double)(b.m - M) * (double)c);
  if (M != M) return LSE{M, __builtin_nan("")};
  return LSE{M, sa + sb};
}
__device__ __forceinline__ LSE wave_lse(LSE v, float c) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    LSE o{__shfl_xor(v.m, m), shfl_xor_f64(v.s, m)};
    v = lse_merge(v, o, c);
  }
  return v;
}

// ---------------------------------------------------------------- workgroup scratch
struct SelShared {
  uint32_t hist[256];
  uint32_t cnt;        // records in the candidate buffer
  uint32_t overflow;   // a tile's candidates did not fit
  uint32_t cnt2;
  uint32_t digit, rem, bcnt;
  uint32_t last;       // this workgroup finishes the row
  uint32_t wtau[NWAVE];
  float wm[NWAVE];
  double ws[NWAVE];
  uint64_t wk[NWAVE];
  uint64_t wk2[NWAVE];
};

// One MSB-first radix step: after `hist` holds the counts of the next 8-bit
// digit among keys matching the prefix, find the digit d holding the rem-th
// largest key.  Wave 0 scans the 256 bins from the top; all threads then read
// (digit, rem within the bucket, bucket count) from sh.
__device__ __forceinline__ void radix_pick(SelShared& sh, uint32_t rem) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    uint32_t c[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) c[b] = sh.hist[255 - 4 * lane - b];
    uint32_t local = c[0] + c[1] + c[2] + c[3];
    uint32_t incl = wave_incl_scan_u32(local, lane);
    uint32_t cum = incl - local;
    if (cum < rem && rem <= incl) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (cum + c[b] >= rem) {
          sh.digit = 255 - 4 * lane - b;
          sh.rem = rem - cum;
          sh.bcnt = c[b];
          break;
        }
        cum += c[b];
      }
    }
  }
}

__device__ __forceinline__ uint64_t wave_and_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v &= shfl_xor_u64(v, m);
  return v;
}
__device__ __forceinline__ uint64_t wave_or_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v |= shfl_xor_u64(v, m);
  return v;
}

// k-th largest of the distinct 64-bit keys produced by `each(f)` (which
// calls f(key) for every key this thread contributes); at least k keys exist.
// Returns T such that exactly k keys are >= T.  MSB-first 8-bit digits; a
// digit on which all keys agree (from the AND / OR of all keys) costs no
// histogram pass.  All threads must call.
template <class Each>
__device__ uint64_t radix_select(SelShared& sh, uint32_t k, Each each) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t all_and = ~0ull, all_or = 0ull;
  each([&](uint64_t K) {
    all_and &= K;
    all_or |= K;
  });
  all_and = wave_and_u64(all_and);
  all_or = wave_or_u64(all_or);
  __syncthreads();
  if (lane == 0) {
    sh.wk[wave] = all_and;
    sh.wk2[wave] = all_or;
  }
  __syncthreads();
  all_and = sh.wk[0];
  all_or = sh.wk2[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) {
    all_and &= sh.wk[q];
    all_or |= sh.wk2[q];
  }
  const uint64_t varies = all_and ^ all_or;
  uint64_t prefix = 0;
  uint32_t rem = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (((varies >> shift) & 0xFFull) == 0) {  // every key has the same digit here
      prefix |= all_and & (0xFFull << shift);
      continue;
    }
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
    const uint64_t hmask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
    each([&](uint64_t K) {
      if ((K & hmask) == prefix) atomicAdd(&sh.hist[(uint32_t)(K >> shift) & 255u], 1u);
    });
    __syncthreads();
    radix_pick(sh, rem);
    __syncthreads();
    prefix |= (uint64_t)sh.digit << shift;
    const uint32_t bc = sh.bcnt;
    rem = sh.rem;
    if (bc == rem) break;  // the whole bucket qualifies
  }
  __syncthreads();
  return prefix;
}

// Shrink the LDS candidate buffer (n > k records) to its k largest keys and
// return the new threshold (the k-th largest key).  `bits` (the records'
// element bits) may be null for a keys-only buffer.  The compaction is done
// in place by wave 0, 64 records at a time: a record's destination (the
// number of winners before it) never lies beyond what the wave has already
// read.  All threads must call.
template <int CAP>
__device__ uint64_t select_compact(SelShared& sh, uint64_t* key, uint32_t* bits, uint32_t n, uint32_t k) {
  const int tid = threadIdx.x;
  const uint64_t T = radix_select(sh, k, [&](auto f) {
    for (uint32_t i = tid; i < n; i += NT) f(key[i]);
  });
  if (tid < 64) {
    uint32_t base = 0;
    for (uint32_t c0 = 0; c0 < n; c0 += 64) {
      const uint32_t i = c0 + tid;
      const uint64_t K = i < n ? key[i] : 0ull;
      const uint32_t b = (bits && i < n) ? bits[i] : 0u;
      const bool win = i < n && K >= T;
      const uint64_t m = __ballot(win);
      if (win) {
        const uint32_t d =
            base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        key[d] = K;
        if (bits) bits[d] = b;
      }
      base += (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  if (tid == 0) sh.cnt = k;
  __syncthreads();
  return T;
}

// Sort key[0..n) (with bits) in descending key order; n <= CAP.
template <int CAP>
__device__ void sort_desc(uint64_t* key, uint32_t* bits, uint32_t n) {
  const int tid = threadIdx.x;
  uint32_t P = 1;
  while (P < n) P <<= 1;
  for (uint32_t i = n + tid; i < P; i += NT) { key[i] = 0ull; bits[i] = 0u; }
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (uint32_t i = tid; i < P / 2; i += NT) {
        uint32_t lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        uint64_t a = key[lo], b = key[hi];
        bool desc = (lo & size) == 0;
        if (desc ? (a < b) : (a > b)) {
          key[lo] = b; key[hi] = a;
          uint32_t t = bits[lo]; bits[lo] = bits[hi]; bits[hi] = t;
        }
      }
    }
  }
  __syncthreads();
}

// The ordered sampler chain on the top-k candidates ("Chapter 21", section
// 21.7: top_n_sigma against the maximum, top_k, typical_p, then the top_p
// nucleus, each over the candidate list; min_p among the filters on the
// untempered distribution and the temperature last, "speculative-acceptance.md",
// "The rules").  key/bits: the n candidates in (value desc, id asc) order, so
// candidate 0 holds the row maximum.
//   top_n_sigma > 0: keep z >= z_0 - n * sigma (a prefix: the list is sorted);
//   typical_p < 1: p over the candidates, H = -sum p log p; reorder by
//     |-log p - H| ascending (ties keep value order), keep the shortest prefix
//     with sum p >= typical_p;
//   top_p < 1: back to value order, keep the shortest prefix with sum p >= top_p
//     (p the softmax of the candidates left);
//   min_p > 0: keep z >= max z + log(min_p) (order unchanged);
//   then w = exp((z - z_0) / T) and the inverse-CDF draw with u in the current
//   order.  logp = log(w_j / sum w).
// All threads call; thread 0 gets tok and logp.  Every sum runs in list order
// on thread 0 (float64), the exponentials, logarithms and typicality ranks run
// in parallel.  Scratch: E and S n doubles, ORD and LIST n words (S and ORD
// only with typical_p < 1).
struct ChainParams {
  float temperature, top_p, top_n_sigma, typical_p, min_p;
  // instead of drawing, the kept set's smallest composite key and log sum of
  // exp(z/T) over it (filtered speculative acceptance; typical_p == 1, so the
  // kept set is a prefix in value order)
  uint64_t* kfl_out;
  double* lse_out;
};
// Lane l's float64 v, in every lane (l uniform).
__device__ __forceinline__ double readlane_f64(double v, uint32_t l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, (int)l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), (int)l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Lane src's value (a gather within the wave).
__device__ __forceinline__ uint32_t from_lane_u32(uint32_t v, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src << 2), (int)v);
}
__device__ __forceinline__ double from_lane_f64(double v, uint32_t src) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = from_lane_u32((uint32_t)b, src), hi = from_lane_u32((uint32_t)(b >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// The lane whose dst is this lane (dst a permutation of the wave's lanes).
__device__ __forceinline__ uint32_t lane_sending_here(uint32_t dst) {
  return (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)(threadIdx.x & 63));
}

// chain_tail (below) for n <= 64 candidates, by wave 0 alone with candidate
// (or list place) l in lane l: the same arithmetic in the same order, every
// in-order sum a loop over the lanes' values read out one by one, so no step
// waits on LDS.  Called by wave 0 only, all its lanes active.
__device__ inline void chain_tail_wave(const uint64_t* key, const uint32_t* bits, uint32_t n, const ChainParams& cp,
                                       double sigma, float u, uint32_t* tok, float* logp) {
  const uint32_t lane = threadIdx.x & 63;
  const bool live = lane < n;
  const double z = live ? (double)__uint_as_float(bits[lane]) : 0.0;
  const double z0 = readlane_f64(z, 0);
  const double e = live ? exp(z - z0) : 0.0;  // E[j]
  uint32_t cnt = n;
  if (cp.top_n_sigma > 0.0f) {
    const double thr = z0 - (double)cp.top_n_sigma * sigma;
    const uint64_t stop = __ballot(lane >= 1 && live && !(z >= thr));
    cnt = stop ? (uint32_t)__builtin_ctzll(stop) : n;
  }
  // the list: place l holds candidate li, its E and its value
  uint32_t li = lane;
  double el = e, zl = z;
  bool value_order = true;
  if (cp.typical_p < 1.0f) {
    const bool in = lane < cnt;
    double Z = 0.0;
    for (uint32_t j = 0; j < cnt; ++j) Z += readlane_f64(e, j);
    const double sj = in && e > 0.0 ? log(e / Z) : -__builtin_inf();
    const double term = (e / Z) * sj;
    double H = 0.0;
    for (uint32_t j = 0; j < cnt; ++j)
      if (readlane_f64(e, j) > 0.0) H -= readlane_f64(term, j);
    const double sc = in && e > 0.0 ? fabs(-sj - H) : __builtin_inf();
    uint32_t r = 0;
    for (uint32_t i = 0; i < cnt; ++i) {
      const double si = readlane_f64(sc, i);
      r += (si < sc || (si == sc && i < lane)) ? 1u : 0u;
    }
    const uint32_t ord = lane_sending_here(in ? r : lane);  // ORD[place]
    const double qv = from_lane_f64(e, ord) / Z;
    double cum = 0.0;
    uint32_t m = cnt;
    for (uint32_t rr = 0; rr < cnt; ++rr) {
      cum += readlane_f64(qv, rr);
      if (cum >= (double)cp.typical_p) {
        m = rr + 1;
        break;
      }
    }
    li = ord;
    el = from_lane_f64(e, ord);
    zl = from_lane_f64(z, ord);
    cnt = m;
    value_order = false;
  }
  if (cp.top_p < 1.0f) {
    if (!value_order) {  // back to value order: candidate indices ascending
      uint32_t rk = 0;
      for (uint32_t i = 0; i < cnt; ++i) rk += (uint32_t)__builtin_amdgcn_readlane((int)li, (int)i) < li ? 1u : 0u;
      const uint32_t src = lane_sending_here(lane < cnt ? rk : lane);
      li = from_lane_u32(li, src);
      el = from_lane_f64(el, src);
      zl = from_lane_f64(zl, src);
      value_order = true;
    }
    double Z = 0.0;
    for (uint32_t i = 0; i < cnt; ++i) Z += readlane_f64(el, i);
    const double qv = el / Z;
    double cum = 0.0;
    for (uint32_t i = 0; i < cnt; ++i) {
      cum += readlane_f64(qv, i);
      if (cum >= (double)cp.top_p) {
        cnt = i + 1;
        break;
      }
    }
  }
  if (cp.min_p > 0.0f) {
    double cmax = readlane_f64(zl, 0);
    if (!value_order)
      for (uint32_t i = 1; i < cnt; ++i) cmax = fmax(cmax, readlane_f64(zl, i));
    const double thr = cmax + log((double)cp.min_p);
    const bool keep = lane < cnt && zl >= thr;
    const uint64_t km = __ballot(keep);
    const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
    const uint32_t nk = (uint32_t)__builtin_popcountll(km);
    const uint32_t src = lane_sending_here(keep ? pos : nk + (lane - pos));  // kept first, in order
    li = from_lane_u32(li, src);
    zl = from_lane_f64(zl, src);
    cnt = nk;
  }
  // the tempered weights, then the draw in list order
  const double T = cp.temperature;
  const double et = lane < cnt ? exp((zl - z0) / T) : 0.0;
  double W = 0.0;
  for (uint32_t i = 0; i < cnt; ++i) W += readlane_f64(et, i);
  if (cp.kfl_out) {
    if (lane == 0) {
      *cp.kfl_out = key[(uint32_t)__builtin_amdgcn_readlane((int)li, (int)(cnt - 1))];
      *cp.lse_out = z0 / T + log(W);
    }
    return;
  }
  const double target = (double)u * W;
  double c = 0.0;
  int pick = -1;
  for (uint32_t i = 0; i < cnt; ++i) {
    c += readlane_f64(et, i);
    if (target < c) {
      pick = (int)i;
      break;
    }
  }
  if (pick < 0) {
    for (int i = (int)cnt - 1; i >= 0; --i)
      if (readlane_f64(et, (uint32_t)i) > 0.0) {
        pick = i;
        break;
      }
    if (pick < 0) pick = 0;
  }
  if (lane == 0) {
    const uint32_t j = (uint32_t)__builtin_amdgcn_readlane((int)li, pick);
    *tok = ~(uint32_t)key[j];
    *logp = (float)(((double)__uint_as_float(bits[j]) - z0) / T - log(W));
  }
}

__device__ inline void chain_tail(const uint64_t* key, const uint32_t* bits, uint32_t n, const ChainParams& cp,
                                  double sigma, float u, double* E, double* S, uint32_t* ORD, uint32_t* LIST,
                                  uint32_t* tok, float* logp) {
  const int tid = threadIdx.x;
  if (n <= 64) {  // (n is uniform) one wave in its lanes; the others are done
    if (tid < 64) chain_tail_wave(key, bits, n, cp, sigma, u, tok, logp);
    return;
  }
  __shared__ uint32_t c_cnt;
  __shared__ double c_Z, c_H;
  auto zv = [&](uint32_t j) { return (double)__uint_as_float(bits[j]); };
  const double z0 = zv(0);
  for (uint32_t j = tid; j < n; j += NT) {
    E[j] = exp(zv(j) - z0);
    LIST[j] = j;
  }
  if (tid == 0) {
    uint32_t n1 = n;
    if (cp.top_n_sigma > 0.0f) {
      const double thr = z0 - (double)cp.top_n_sigma * sigma;
      n1 = 1;
      while (n1 < n && zv(n1) >= thr) ++n1;
    }
    c_cnt = n1;
  }
  __syncthreads();
  uint32_t cnt = c_cnt;
  bool value_order = true;
  if (cp.typical_p < 1.0f) {
    if (tid == 0) {
      double Z = 0.0;
      for (uint32_t j = 0; j < cnt; ++j) Z += E[j];
      c_Z = Z;
    }
    __syncthreads();
    const double Z = c_Z;
    for (uint32_t j = tid; j < cnt; j += NT) S[j] = E[j] > 0.0 ? log(E[j] / Z) : -__builtin_inf();
    __syncthreads();
    if (tid == 0) {
      double H = 0.0;
      for (uint32_t j = 0; j < cnt; ++j)
        if (E[j] > 0.0) H -= (E[j] / Z) * S[j];
      c_H = H;
    }
    __syncthreads();
    const double H = c_H;
    for (uint32_t j = tid; j < cnt; j += NT) S[j] = E[j] > 0.0 ? fabs(-S[j] - H) : __builtin_inf();
    __syncthreads();
    for (uint32_t j = tid; j < cnt; j += NT) {
      const double sj = S[j];
      uint32_t r = 0;
      for (uint32_t i = 0; i < cnt; ++i) r += (S[i] < sj || (S[i] == sj && i < j)) ? 1u : 0u;
      ORD[r] = j;
    }
    __syncthreads();
    if (tid == 0) {
      double cum = 0.0;
      uint32_t m = cnt;
      for (uint32_t r = 0; r < cnt; ++r) {
        cum += E[ORD[r]] / Z;
        if (cum >= (double)cp.typical_p) {
          m = r + 1;
          break;
        }
      }
      for (uint32_t r = 0; r < m; ++r) LIST[r] = ORD[r];
      c_cnt = m;
    }
    __syncthreads();
    cnt = c_cnt;
    value_order = false;
  }
  if (tid == 0) {
    if (cp.top_p < 1.0f) {
      if (!value_order)  // back to value order: candidate indices ascending
        for (uint32_t i = 1; i < cnt; ++i) {
          const uint32_t v = LIST[i];
          uint32_t j = i;
          for (; j > 0 && LIST[j - 1] > v; --j) LIST[j] = LIST[j - 1];
          LIST[j] = v;
        }
      value_order = true;
      double Z = 0.0;
      for (uint32_t i = 0; i < cnt; ++i) Z += E[LIST[i]];
      double cum = 0.0;
      for (uint32_t i = 0; i < cnt; ++i) {
        cum += E[LIST[i]] / Z;
        if (cum >= (double)cp.top_p) {
          cnt = i + 1;
          break;
        }
      }
    }
    if (cp.min_p > 0.0f) {
      double cmax = zv(LIST[0]);
      if (!value_order)
        for (uint32_t i = 1; i < cnt; ++i) cmax = fmax(cmax, zv(LIST[i]));
      const double thr = cmax + log((double)cp.min_p);
      uint32_t m = 0;
      for (uint32_t i = 0; i < cnt; ++i)
        if (zv(LIST[i]) >= thr) LIST[m++] = LIST[i];
      cnt = m;
    }
    c_cnt = cnt;
  }
  __syncthreads();
  cnt = c_cnt;
  // the tempered weights (E is free now), then the draw in list order
  const double T = cp.temperature;
  for (uint32_t i = tid; i < cnt; i += NT) E[i] = exp((zv(LIST[i]) - z0) / T);
  __syncthreads();
  if (tid == 0 && cp.kfl_out) {
    double W = 0.0;
    for (uint32_t i = 0; i < cnt; ++i) W += E[i];
    *cp.kfl_out = key[LIST[cnt - 1]];
    *cp.lse_out = z0 / T + log(W);
  } else if (tid == 0) {
    double W = 0.0;
    for (uint32_t i = 0; i < cnt; ++i) W += E[i];
    const double target = (double)u * W;
    double c = 0.0;
    int pick = -1;
    for (uint32_t i = 0; i < cnt; ++i) {
      c += E[i];
      if (target < c) {
        pick = (int)i;
        break;
      }
    }
    if (pick < 0) {
      for (int i = (int)cnt - 1; i >= 0; --i)
        if (E[i] > 0.0) {
          pick = i;
          break;
        }
      if (pick < 0) pick = 0;
    }
    const uint32_t j = LIST[pick];
    *tok = ~(uint32_t)key[j];
    *logp = (float)((zv(j) - z0) / T - log(W));
  }
}

// A value every lane of the wave holds, kept in scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// One full tile of NG 16-byte groups per lane through a buffer resource
// based at the tile (scalar base, per-lane offset, per-group scalar offset:
// no vector address arithmetic); reads past the tile would return zero.
template <typename DT, int NG>
__device__ __forceinline__ void load_tile_buf(Group (&g)[NG], const DT* __restrict__ tb) {
  constexpr int E = Elem<DT>::E;
  constexpr int kTileBytes = NT * NG * 16;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)tb, 0, kTileBytes, 0x00020000);
  const int vo = (int)threadIdx.x * 16;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, j * NT * 16, 2 /* nontemporal */);
    g[j].w[0] = v.x; g[j].w[1] = v.y; g[j].w[2] = v.z; g[j].w[3] = v.w;
  }
  (void)E;
}

// A row's last, partial tile by the same buffer loads, all issued together:
// lim (uniform) is the number of elements left from tb, a multiple of E and
// at least E.  Groups at or past lim read as -inf; their lanes re-read the
// tile's first group, so every address lies inside the row.  (The lane
// offsets are formed here, from a thread index the compiler cannot hoist,
// so no per-lane constant of this rare tile stays live through the loop.)
template <typename DT, int NG>
__device__ __forceinline__ void load_tile_buf_part(Group (&g)[NG], const DT* __restrict__ tb, uint32_t lim) {
  constexpr int E = Elem<DT>::E;
  constexpr uint32_t pad = (E == 4) ? kNegInfBits : 0xFF80FF80u;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)tb, 0, (int)(lim * (uint32_t)sizeof(DT)), 0x00020000);
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const uint32_t o = ((uint32_t)j * NT + tid) * E;
    const bool full = o < lim;
    const u32x4 v =
        __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((full ? o : 0u) * (uint32_t)sizeof(DT)), 0, 2 /* nontemporal */);
    g[j].w[0] = full ? v.x : pad;
    g[j].w[1] = full ? v.y : pad;
    g[j].w[2] = full ? v.z : pad;
    g[j].w[3] = full ? v.w : pad;
  }
}

// 2^a in float64 for a finite a, to float precision (the fraction through
// the hardware exp2, the integer part exactly through ldexp); saturates far
// outside the float64 range.
__device__ __forceinline__ double exp2_split(double a) {
  a = fmin(fmax(a, -1100.0), 1100.0);
  const double n = floor(a);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(a - n)), (int)n);
}

// e^x in float64 for x <= 0 (0 below -745).  x = k ln2/64 + r, the reduction
// with ln2/64 split in two (the high part has 25 significant bits, so k * hi
// is exact for the k that occur); e^r by its Taylor series to r^6 (|r| <=
// ln2/128, so the truncation is below 1e-19); then 2^(k/64) as a table entry
// 2^((k mod 64)/64) and an exponent shift.  A few units in the last place,
// like a library exp.  Host code may call it too (with the table filled by
// the host's exp2), which is how it is checked against a high-precision
// exponential.
constexpr double kL64Hi = 0x1.62e42f0000000p-7;   // ln2/64, high part
constexpr double kL64Lo = 0x1.df473de6af279p-32;  // ln2/64 - kL64Hi
constexpr double kInvL64 = 0x1.71547652b82fep+6;  // 64/ln2
__host__ __device__ __forceinline__ double exp_le0(double x, const double* e2) {
  const double xc = fmax(x, -745.0);
  const double k = rint(xc * kInvL64);
  const double r = fma(-k, kL64Lo, fma(-k, kL64Hi, xc));
  double p = fma(r, 1.0 / 720.0, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ki = (int)k;
  const double v = ldexp(e2[ki & 63] * p, ki >> 6);
  return x < -745.0 ? 0.0 : v;
}

// The table 2^(j/64), j = 0..63, in LDS (all threads call).
__device__ __forceinline__ void init_e2(double* e2) {
  if (threadIdx.x < 64) e2[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
  __syncthreads();
}

// Log-sum-exp states (m, s) of the workgroup's lanes merged: the maximum
// first (NaN-propagating), then one rescale per lane and float64 sums, so
// no step pays more than one exp2.  Every thread must call; every thread
// gets the result.
__device__ __forceinline__ LSE block_lse(LSE v, float c, float* sm, double* ss) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float M = wave_max_nan(v.m);
  if (lane == 0) sm[wave] = M;
  __syncthreads();
  M = sm[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) M = fmax_nan(M, sm[q]);
  double t = 0.0;
  if (M != M || M == __builtin_inff()) t = __builtin_nan("");
  else if (v.m != -__builtin_inff()) t = v.s * exp2_split(((double)v.m - (double)M) * (double)c);
  t = wave_sum_f64(t);
  if (lane == 0) ss[wave] = t;
  __syncthreads();
  double S = ss[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) S += ss[q];
  return LSE{M, S};
}

// Cross-workgroup data (segment partials, tickets) moves only through
// device-scope atomic loads and stores.  On gfx950 these are coherent across
// the XCDs' separate L2s by themselves, so no whole-cache writeback or
// invalidate is needed (an agent-scope fence would cost one per workgroup).
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) { st_dev(reinterpret_cast<uint32_t*>(p), (uint32_t)v); }
__device__ __forceinline__ void st_dev(float* p, float v) { st_dev(reinterpret_cast<uint32_t*>(p), __float_as_uint(v)); }
__device__ __forceinline__ void st_dev(double* p, double v) {
  st_dev(reinterpret_cast<uint64_t*>(p), (uint64_t)__double_as_longlong(v));
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(ld_dev(reinterpret_cast<const uint32_t*>(p)));
}
__device__ __forceinline__ double ld_dev(const double* p) {
  return __longlong_as_double((long long)ld_dev(reinterpret_cast<const uint64_t*>(p)));
}

// Last-workgroup-done ticket.  Every thread has written its partial results
// with st_dev; waiting for its outstanding memory operations makes them
// complete at device scope before the workgroup's arrival is counted.
// Returns true in exactly one of the `n` workgroups sharing `ticket` (the
// last to arrive), which may then read every partial with ld_dev; it resets
// the ticket to 0 for the next call.  All threads must call.
__device__ __forceinline__ bool last_done(SelShared& sh, uint32_t* ticket, uint32_t n) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = (old == n - 1) ? 1u : 0u;
    if (old == n - 1) st_dev(ticket, 0u);
  }
  __syncthreads();
  return sh.last != 0;
}

// ---------------------------------------------------------------- moments
// (count, mean, squared deviations) of a set of values; two sets merge by the
// pairwise update of Chan, Golub and LeVeque.
struct Mom {
  double n, mean, m2;
};

__device__ __forceinline__ Mom mom_merge(Mom a, Mom b) {
  if (b.n == 0.0) return a;
  if (a.n == 0.0) return b;
  const double n = a.n + b.n, d = b.mean - a.mean;
  return Mom{n, a.mean + d * (b.n / n), a.m2 + b.m2 + d * d * (a.n * b.n / n)};
}

// Lanes folded into lane 0 in a fixed order (lane l takes lane l + 2^s).
__device__ __forceinline__ Mom wave_mom(Mom v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const Mom o{__shfl_down(v.n, d), __shfl_down(v.mean, d), __shfl_down(v.m2, d)};
    if (((int)(threadIdx.x & 63) & (2 * d - 1)) == 0) v = mom_merge(v, o);
  }
  return v;  // lane 0
}

// ---------------------------------------------------------------- merges
// Reductions over per-segment partials, loaded in parallel (one thread per
// segment) so that their device-scope load latencies overlap.  S <= NT.
__device__ __forceinline__ double block_sum_f64(SelShared& sh, double v) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) sh.ws[wave] = v;
  __syncthreads();
  double t = sh.ws[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) t += sh.ws[q];
  return t;
}

// Sum of p[0..S) (all threads get it; fixed order for a given S).
__device__ __forceinline__ double merge_sum(SelShared& sh, const double* p, int S) {
  const int tid = threadIdx.x;
  return block_sum_f64(sh, tid < S ? ld_dev(&p[tid]) : 0.0);
}

// Combined (key max, log-sum-exp) of S partials (all threads get them).
__device__ __forceinline__ void merge_key_lse(SelShared& sh, const uint64_t* pk, const float* pm, const double* ps,
                                              int S, float c, uint64_t& P, LSE& r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t k = 0;
  LSE v{-__builtin_inff(), 0.0};
  if (tid < S) {
    if (pk) k = ld_dev(&pk[tid]);
    v = LSE{ld_dev(&pm[tid]), ld_dev(&ps[tid])};
  }
  // The maximum first (NaN-propagating), then every partial rescaled to it at
  // once (one float64 exp2 per lane, not a chain of pairwise merges) and
  // summed in a fixed order.
  k = wave_max_u64(k);
  float M = wave_max_nan(v.m);
  __syncthreads();
  if (lane == 0) {
    sh.wk[wave] = k;
    sh.wm[wave] = M;
  }
  __syncthreads();
  P = sh.wk[0];
  M = sh.wm[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) {
    P = sh.wk[q] > P ? sh.wk[q] : P;
    M = fmax_nan(M, sh.wm[q]);
  }
  double t = 0.0;
  if (v.m == M) t = v.s;
  else if (v.m != -__builtin_inff()) t = v.s * exp2((double)(v.m - M) * (double)c);
  t = wave_sum_f64(t);
  if (lane == 0) sh.ws[wave] = t;
  __syncthreads();
  double sum = sh.ws[0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) sum += sh.ws[q];
  r = (M != M) ? LSE{M, __builtin_nan("")} : LSE{M, sum};
}

// Work index of this workgroup, remapped so that consecutive work items run
// on the same XCD (workgroups are dealt round-robin over the 8 XCDs), which
// keeps the segments of one row and their partials in one L2.
__device__ __forceinline__ uint32_t work_index() {
  const uint32_t b = blockIdx.x, n = gridDim.x;
  if ((n & 7u) == 0) return (b & 7u) * (n >> 3) + (b >> 3);
  return b;
}

// (row, segment) of this workgroup's work item, computed in 32 bits and kept
// uniform.
struct Item {
  uint32_t row, seg;
};
__device__ __forceinline__ Item work_item(int32_t S) {
  const uint32_t w = work_index();
  const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(w / (uint32_t)S);
  return Item{row, (uint32_t)__builtin_amdgcn_readfirstlane(w - row * (uint32_t)S)};
}

}  // namespace vsel
