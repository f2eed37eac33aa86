// index_common.h -- device helpers shared by the indexer kernels (index_topk.hip, index_cand.hip).
#pragma once

#include "csah_internal.h"
#include "device_common.h"

namespace csah {

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kBins = 4096;
constexpr int kBinShift = 20;  // top 12 bits of the order key
// Scores of the decode scan are staged in LDS and written out a window at a time: stores mixed
// into the key stream cost about 10% of the scan's time, one burst per window much less. The
// window is capped so that a CU holding two scan workgroups (16 KB histogram + 16 KB stage
// each) still has LDS for an attention workgroup running concurrently on another stream; with
// 32 KB windows that co-residency is lost and two-layer decode steps get about 10% slower.
constexpr int kScoreStage = 4096;

__device__ __forceinline__ int64_t visible_entries(const int64_t* pos, int b, int i, int m,
                                                   int64_t N) {
  int64_t nv = (pos[b] + i + 1) / m;
  return nv < 0 ? 0 : (nv > N ? N : nv);
}

// dI/32 consecutive lanes score one entry, one 32-element block each: a wavefront's 16-byte loads
// cover one contiguous kilobyte of codes. Each lane holds its block's 32 head-summed query values.
template <int NB>
__device__ __forceinline__ float block_score(const u32x4 c, uint32_t e, const float* qv) {
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const f32x2 v0 = fp4x2_to_f32<0>(c[j]);
    const f32x2 v1 = fp4x2_to_f32<1>(c[j]);
    const f32x2 v2 = fp4x2_to_f32<2>(c[j]);
    const f32x2 v3 = fp4x2_to_f32<3>(c[j]);
    t = fmaf(v0[0], qv[8 * j + 0], t);
    t = fmaf(v0[1], qv[8 * j + 1], t);
    t = fmaf(v1[0], qv[8 * j + 2], t);
    t = fmaf(v1[1], qv[8 * j + 3], t);
    t = fmaf(v2[0], qv[8 * j + 4], t);
    t = fmaf(v2[1], qv[8 * j + 5], t);
    t = fmaf(v3[0], qv[8 * j + 6], t);
    t = fmaf(v3[1], qv[8 * j + 7], t);
  }
  // times 2^(E-127): exact (the block sum is a multiple of a power of two well inside range)
  float s = ldexpf(t, (int)e - 127);
  if constexpr (NB >= 2) s = quad_xor1_add(s);
  if constexpr (NB >= 4) s = quad_xor2_add(s);
  return s + 0.0f;  // fold -0 into +0: equal scores must get equal keys
}

// Paged keys: a workgroup first copies the block-table entries of the pages its keys span into
// LDS, so each row's pool address costs an LDS read instead of a dependent global load.
constexpr int kPageList = 1040;  // the host sizes key ranges to span at most 1026 pages

// Page list of sequence b's entries [g0, g1) (g0 < g1) into LDS; every thread takes part.
__device__ __forceinline__ void load_page_list(const EntryMap& km, int b, int64_t g0, int64_t g1,
                                               int32_t* pages, int tid, int nthreads) {
  const int64_t p0 = g0 >> km.shift;
  const int np = (int)(((g1 - 1) >> km.shift) - p0 + 1);
  const int32_t* t = km.table + (int64_t)b * km.stride + p0;
  for (int j = tid; j < np; j += nthreads) pages[j] = t[j];
}

// Pool row of the entry at offset rr from the start of the first listed page.
__device__ __forceinline__ uint64_t page_row(const int32_t* pages, uint32_t rr, int shift) {
  return ((uint64_t)(uint32_t)pages[rr >> shift] << shift) | (rr & ((1u << shift) - 1u));
}

// DPP quad permute of a float (every lane reads a lane of its own quad).
template <int CTRL>
__device__ __forceinline__ float quad_read(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// ---- scaled-FP4 MFMA scoring of 16 keys against 16 queries (one indexer head per product) ----
template <int HP>  // HP >= HI: heads padded with zero codes contribute exactly 0
struct QueryOps {
  i32x8 c[HP];
  int e[HP];
};

template <int HP>
__device__ __forceinline__ void load_query_ops(const uint8_t* __restrict__ q_codes,
                                               const uint8_t* __restrict__ q_scales, int HI,
                                               int64_t qrow, bool valid, int blk, QueryOps<HP>& o) {
#pragma unroll
  for (int h = 0; h < HP; h++) {
    o.c[h] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    o.e[h] = 127;
    if (valid && h < HI) {
      const u32x4 v = *(const u32x4*)(q_codes + (qrow * HI + h) * 64 + 16 * blk);
      o.c[h][0] = (int)v[0];
      o.c[h][1] = (int)v[1];
      o.c[h][2] = (int)v[2];
      o.c[h][3] = (int)v[3];
      o.e[h] = q_scales[(qrow * HI + h) * 4 + blk];
    }
  }
}

template <int HP>
__device__ __forceinline__ f32x4 tile_scores(const u32x4 kc, uint32_t ke, const QueryOps<HP>& o) {
  const i32x8 a = i32x8{(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < HP; h++)
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, o.c[h], acc, 4, 4, 0, (int)ke, 0,
                                                           o.e[h]);
  return acc;
}

// Walk over a workgroup's keys: each wavefront takes every 4th tile of 16 keys. Loads go
// in rounds of U tiles, double-buffered, so one round's loads are in flight while the previous
// round is scored; `visit(key, scores, n)` sees the lane's query scored against the four
// consecutive keys from `key` on, of which the first n (n >= 1) are visible.
// Paged keys: `pages` (LDS, kPageList entries) receives the range's block-table entries; the
// walk's early return is uniform over the workgroup, so the barrier after filling it is safe.
// The keys [g0, gend) of sequence b (cut at the block's visible keys) against query block qb.
template <int HP, bool PAGED, typename F>
__device__ __forceinline__ void mfma_walk_keys(const uint8_t* __restrict__ q_codes,
                                               const uint8_t* __restrict__ q_scales, int HI,
                                               const uint8_t* __restrict__ k_codes,
                                               const uint8_t* __restrict__ k_scales,
                                               const EntryMap& kmap, int64_t N,
                                               const int64_t* __restrict__ pos, int m, int Q,
                                               int b, int qb, int64_t g0, int64_t gend,
                                               int32_t* pages, F visit) {
  constexpr int U = 4;
  const int q0 = qb * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, blk = lane >> 4;
  const int qi = q0 + n;
  const bool qv = qi < Q;
  const int64_t nv = qv ? visible_entries(pos, b, qi, m, N) : 0;
  // visibility is nondecreasing in the query index: the block's last query sees the most
  const int64_t nvmax = visible_entries(pos, b, (q0 + 15 < Q ? q0 + 15 : Q - 1), m, N);
  const int64_t g1 = gend < nvmax ? gend : nvmax;
  if (g0 >= g1) return;
  if constexpr (PAGED) {
    load_page_list(kmap, b, g0, g1, pages, threadIdx.x, 256);
    __syncthreads();
  }
  QueryOps<HP> qo;
  load_query_ops<HP>(q_codes, q_scales, HI, (int64_t)b * Q + qi, qv, blk, qo);
  const int64_t base_row = PAGED ? 0 : kmap.row(b, g0);
  const uint8_t* kc = k_codes + base_row * 64 + 16 * blk;
  const uint8_t* ks = k_scales + base_row * 4 + blk;
  const uint32_t off0 = PAGED ? (uint32_t)(g0 & (((int64_t)1 << kmap.shift) - 1)) : 0u;
  const int nk = (int)(g1 - g0);
  const int ntile = (nk + 15) / 16;
  const int my_tiles = ntile > wave ? (ntile - wave + 3) / 4 : 0;  // tiles wave, wave+4, ...
  auto load = [&](int j0, u32x4* c, uint32_t* e) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      int r = 16 * (wave + 4 * (j0 + u)) + n;  // key row of this lane in the A operand
      r = r < nk ? r : nk - 1;                 // rows past the range read a valid row (masked)
      if constexpr (PAGED) {
        const uint64_t row = page_row(pages, off0 + (uint32_t)r, kmap.shift);
        c[u] = __builtin_nontemporal_load((const u32x4*)(kc + row * 64u));
        e[u] = ks[row * 4u];
      } else {
        c[u] = __builtin_nontemporal_load((const u32x4*)(kc + (uint32_t)r * 64u));
        e[u] = ks[(uint32_t)r * 4u];
      }
    }
  };
  // keys of this lane's query that are visible, relative to g0 (so compares are 32-bit)
  const int lim = (int)((nv < g1 ? nv : g1) - g0 > 0 ? (nv < g1 ? nv : g1) - g0 : 0);
  auto score = [&](int j0, const u32x4* c, const uint32_t* e) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (j0 + u >= my_tiles) break;
      f32x4 sc = tile_scores<HP>(c[u], e[u], qo);
      const int kr0 = 16 * (wave + 4 * (j0 + u)) + 4 * blk;
      const int nvis = lim - kr0 < 0 ? 0 : (lim - kr0 > 4 ? 4 : lim - kr0);
#pragma unroll
      for (int i = 0; i < 4; i++) sc[i] += 0.0f;  // fold -0 into +0
      if (nvis > 0) visit(g0 + kr0, sc, nvis);
    }
  };
  u32x4 ca[U], cb[U];
  uint32_t ea[U], eb[U];
  if (my_tiles > 0) load(0, ca, ea);
  for (int j = 0; j < my_tiles; j += 2 * U) {
    if (j + U < my_tiles) load(j + U, cb, eb);
    score(j, ca, ea);
    if (j + U >= my_tiles) break;
    if (j + 2 * U < my_tiles) load(j + 2 * U, ca, ea);
    score(j + U, cb, eb);
  }
}

}  // namespace csah
