// index_rank.h -- workgroup-wide ranking helpers of the indexer kernels (index_cand.hip,
// index_topk.hip): wavefront scans and maxima on DPP, block reductions, stable compaction of
// register-held keys, and a bucket ranking of unique 64-bit keys in descending order.
#pragma once

#include "index_common.h"

namespace csah {

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// ---- wavefront scans on DPP -------------------------------------------------------------------
// Row shifts by 1, 2, 4 and 8 give every lane the inclusive scan of its 16-lane row; broadcasting
// lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3, extends it to the whole wavefront.
// Lanes whose source lies outside the row, and rows the mask leaves out, take the identity.
__device__ __forceinline__ uint32_t wave_prefix_add(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}

// Inclusive scan within each 16-lane row (lane 15 of a row ends with the row's sum).
__device__ __forceinline__ uint32_t row_prefix_add(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
  return v;
}

// Maximum over the wavefront (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// 64-bit maximum over the wavefront: the high words first, then the low words of the lanes that
// hold the largest high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t h = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t l = wave_max_u32((uint32_t)(v >> 32) == h ? (uint32_t)v : 0u);
  return ((uint64_t)h << 32) | l;
}

// ---- block-wide helpers (all NT threads of the workgroup call them) ----------------------------
template <int NT>
struct Blk {
  static constexpr int NW = NT / 64;
  // lanes below this one in the wavefront whose bit of m is set
  static __device__ __forceinline__ uint32_t below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  }
  static __device__ __forceinline__ uint32_t sum(uint32_t v) {
    __shared__ uint32_t s_w[NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_add(v), 63);
    if (lane == 0) s_w[wave] = v;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) r += s_w[w];
    __syncthreads();
    return r;
  }
  static __device__ __forceinline__ uint64_t max64(uint64_t v) {
    __shared__ uint64_t s_w[NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_u64(v);
    if (lane == 0) s_w[wave] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) r = max_u64(r, s_w[w]);
    __syncthreads();
    return r;
  }
  // (min of a, max of b) over the workgroup, one exchange
  static __device__ __forceinline__ void minmax32(uint32_t a, uint32_t b, uint32_t* mn,
                                                  uint32_t* mx) {
    __shared__ uint32_t s_a[NW], s_b[NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = ~wave_max_u32(~a);
    b = wave_max_u32(b);
    if (lane == 0) {
      s_a[wave] = a;
      s_b[wave] = b;
    }
    __syncthreads();
    uint32_t ra = 0xFFFFFFFFu, rb = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      ra = min(ra, s_a[w]);
      rb = max(rb, s_b[w]);
    }
    __syncthreads();
    *mn = ra;
    *mx = rb;
  }
  static __device__ __forceinline__ uint32_t max32(uint32_t v) {
    __shared__ uint32_t s_w[NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_u32(v);
    if (lane == 0) s_w[wave] = v;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) r = max(r, s_w[w]);
    __syncthreads();
    return r;
  }
  // The bin holding the r-th largest counted item of an nb-bin LDS histogram (bin order = item
  // order): *bin, and *above = the count in the higher bins; returns the total count (when it is
  // below r, *bin and *above are not set).
  static __device__ __forceinline__ uint32_t find_bin(const uint32_t* hist, int nb, uint32_t r,
                                                      uint32_t* bin, uint32_t* above) {
    __shared__ uint32_t s_w[NW];
    __shared__ uint32_t s_bin, s_above;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int per = (nb + NT - 1) / NT;
    const int lo = t * per;
    uint32_t v = 0;
    for (int j = 0; j < per; j++) v += lo + j < nb ? hist[lo + j] : 0u;
    const uint32_t pre = wave_prefix_add(v);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63);
    if (lane == 0) s_w[wave] = wtot;
    __syncthreads();
    uint32_t above_w = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      above_w += w > wave ? s_w[w] : 0u;
      total += s_w[w];
    }
    const uint32_t suf = above_w + wtot - pre + v;  // items in this thread's bins and above
    const uint32_t next = suf - v;                  // items above this thread's bins
    if (suf >= r && next < r) {  // exactly one thread: the suffix count crosses r here
      uint32_t acc = next, bsel = (uint32_t)lo;
      for (int j = per - 1; j >= 0; j--) {
        const uint32_t c = lo + j < nb ? hist[lo + j] : 0u;
        if (acc + c >= r) {
          bsel = (uint32_t)(lo + j);
          break;
        }
        acc += c;
      }
      s_bin = bsel;
      s_above = acc;
    }
    __syncthreads();
    *bin = s_bin;
    *above = s_above;
    return total;
  }
  // Exclusive suffix sums of an nb-bin LDS histogram into out[b] = sum of cnt[b'] for b' > b
  // (the start of bin b when the bins are laid out from the top down).
  static __device__ __forceinline__ void suffix_starts(const uint32_t* cnt, int nb, uint32_t* out) {
    __shared__ uint32_t s_w[NW];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int per = (nb + NT - 1) / NT;
    const int lo = t * per;
    uint32_t v = 0;
    for (int j = 0; j < per; j++) v += lo + j < nb ? cnt[lo + j] : 0u;
    const uint32_t pre = wave_prefix_add(v);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63);
    if (lane == 0) s_w[wave] = wtot;
    __syncthreads();
    uint32_t above = wtot - pre;  // bins of the higher threads of this wavefront
#pragma unroll
    for (int w = 0; w < NW; w++) above += w > wave ? s_w[w] : 0u;
    for (int j = per - 1; j >= 0; j--) {
      if (lo + j < nb) {
        out[lo + j] = above;
        above += cnt[lo + j];
      }
    }
    __syncthreads();
  }
};

// Keys held in registers, KPT per thread: key j of thread t is item t + NT * j (0 = no key).

// Stable compaction of the register-held keys (item t + NT * j, considered while below n) for
// which keep(x) holds into out[base..), in item order. Returns how many were kept.
template <int NT, int KPT, typename F>
__device__ __forceinline__ int compact_regs(const uint64_t (&x)[KPT], int n, F keep,
                                            uint64_t* out, int base) {
  typedef Blk<NT> B;
  constexpr int NW = NT / 64, NC = KPT * NW;
  static_assert(NC <= 128, "one wavefront scans the counts, two per lane");
  __shared__ uint32_t s_cnt[NC];
  __shared__ uint32_t s_total;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint64_t m[KPT];
#pragma unroll
  for (int j = 0; j < KPT; j++) {
    const bool f = t + NT * j < n && keep(x[j]);
    m[j] = __ballot(f);
    if (lane == 0) s_cnt[j * NW + wave] = (uint32_t)__popcll(m[j]);
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of the counts in (j, wavefront) order, which is item order
    const uint32_t c0 = 2 * lane < NC ? s_cnt[2 * lane] : 0u;
    const uint32_t c1 = 2 * lane + 1 < NC ? s_cnt[2 * lane + 1] : 0u;
    const uint32_t incl = wave_prefix_add(c0 + c1);
    const uint32_t ex = incl - c0 - c1;
    if (2 * lane < NC) s_cnt[2 * lane] = ex;
    if (2 * lane + 1 < NC) s_cnt[2 * lane + 1] = ex + c0;
    if (lane == 63) s_total = incl;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; j++)
    if ((m[j] >> lane) & 1) out[base + (int)s_cnt[j * NW + wave] + (int)B::below(m[j])] = x[j];
  const int total = (int)s_total;
  __syncthreads();
  return total;
}

// Load items [0, n) of an LDS key array into the register layout of compact_regs / top_sorted.
template <int NT, int KPT>
__device__ __forceinline__ void load_regs(const uint64_t* buf, int n, uint64_t (&x)[KPT]) {
#pragma unroll
  for (int j = 0; j < KPT; j++) {
    const int at = (int)threadIdx.x + NT * j;
    x[j] = at < n ? buf[at] : 0;
  }
}

// Ranks the nonzero register-held keys (distinct) in descending order, writes the first kk of
// them (io[rank], so[rank]) and returns the kk-th largest (1 when there are fewer than kk: then all
// are written). A bucket sort from the top: bins fitted to the keys' range (whole high words), so
// they spread over up to 4096 bins; a key's rank is its bin's start (the count in the higher bins)
// plus the larger keys in its own bin, which holds few. cnt and cur are 4096-entry LDS arrays,
// sorted an LDS array with room for every key held.
template <int NT, int KPT>
__device__ uint64_t top_sorted(const uint64_t (&x)[KPT], uint32_t kk, uint32_t* cnt,
                               uint32_t* cur, uint64_t* sorted, int32_t* __restrict__ io,
                               float* __restrict__ so) {
  typedef Blk<NT> B;
  __shared__ uint64_t s_T;
  const int t = threadIdx.x;
  uint32_t lh = 0xFFFFFFFFu, hh = 0;
#pragma unroll
  for (int j = 0; j < KPT; j++)
    if (x[j] != 0) {
      lh = min(lh, (uint32_t)(x[j] >> 32));
      hh = max(hh, (uint32_t)(x[j] >> 32));
    }
  B::minmax32(lh, hh, &lh, &hh);
  if (t == 0) s_T = 1;
  if (lh > hh) {  // no key at all
    __syncthreads();
    return 1;
  }
  uint64_t base = (uint64_t)lh << 32;
  uint64_t span = ((((uint64_t)hh) << 32) | 0xFFFFFFFFull) - base;
  if (lh == hh) {  // one score (ties everywhere): fit the bins to the low words instead
    uint32_t ll = 0xFFFFFFFFu, hl = 0;
#pragma unroll
    for (int j = 0; j < KPT; j++)
      if (x[j] != 0) {
        ll = min(ll, (uint32_t)x[j]);
        hl = max(hl, (uint32_t)x[j]);
      }
    B::minmax32(ll, hl, &ll, &hl);
    base |= ll;
    span = hl - ll;
  }
  const int bits = span ? 64 - __clzll((long long)span) : 0;
  const int s = bits > 12 ? bits - 12 : 0;
  const int nb = (int)(span >> s) + 1;
  for (int j = t; j < nb; j += NT) cnt[j] = 0u;
  __syncthreads();
  uint32_t bn[KPT];
#pragma unroll
  for (int j = 0; j < KPT; j++) {
    bn[j] = (uint32_t)((x[j] - base) >> s);
    if (x[j] != 0) atomicAdd(&cnt[bn[j]], 1u);
  }
  __syncthreads();
  B::suffix_starts(cnt, nb, cur);
  uint32_t at[KPT];
#pragma unroll
  for (int j = 0; j < KPT; j++)
    if (x[j] != 0) at[j] = atomicAdd(&cur[bn[j]], 1u);
#pragma unroll
  for (int j = 0; j < KPT; j++)
    if (x[j] != 0) sorted[at[j]] = x[j];
  __syncthreads();
  // cur[b] is now the end of bin b, which starts at cur[b] - cnt[b]. The keys that can rank
  // below kk sit at the positions before the end of the bin holding position kk - 1 (all of them,
  // when there are fewer keys): one or two per thread.
  const uint32_t total = cur[0];  // bin 0 ends at the last position
  uint32_t lim = total;
  if (kk < total) lim = cur[(uint32_t)((sorted[kk - 1] - base) >> s)];
  for (uint32_t p = t; p < lim; p += NT) {
    const uint64_t y = sorted[p];
    const uint32_t b = (uint32_t)((y - base) >> s);
    const uint32_t e = cur[b], st = e - cnt[b];
    uint32_t rank = st;
    for (uint32_t q = st; q < e; q++) rank += sorted[q] > y ? 1u : 0u;
    if (rank < kk) {
      io[rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)y);
      if (so) so[rank] = key_to_float((uint32_t)(y >> 32));
      if (rank == kk - 1) s_T = y;
    }
  }
  __syncthreads();
  const uint64_t T = s_T;
  __syncthreads();
  return T;
}

}  // namespace csah
