// index_cand.hip -- decode indexer (one or two queries per sequence, and 3 to 7 with 128-dim keys):
// a scan that leaves certified per-range candidate lists, then one exact top-k over their union.
// With several queries per sequence one scan workgroup scores its range for all of them at once
// (the multi-query MFMA tiles) and publishes a list per query (index_cand_mq_scan_kernel).
//
// [EXPL] "DeepSeek V4 Architecture Explained: CSA, HCA, mHC and Muon", section "How
// compress-then-sparsify attention works": the indexer queries are scored against the compressed
// indexer keys and each query keeps its top-k entries. [LLMB] "Inside DeepSeek-V4 ...", section
// "1. Compressed Sparse Attention (CSA)": an FP4 indexer scores every compressed block and keeps
// the top 1,024. [BSWEN] "How DeepSeek V4 Handles 1M Token Context with Hybrid Attention", section
// "Component 3: DeepSeek Sparse Attention (DSA)": score all entries, keep the top k, attend.
//
// Key of entry g: order_key(score_g) << 32 | ~g. Keys are unique and a larger key means a higher
// score, or an equal score and a lower index, so the output (score descending, index ascending) is
// the kk = min(k, visible) largest keys in descending order.
//
// scan (grid: ranges x slots). A workgroup scores the visible keys of one range of at most 4096
//   entries into LDS and counts a 4096-bin histogram of the top 12 bits of their keys. It then
//   publishes a list P of its keys and a bound u that is at least every key it did not publish:
//   P = the keys of the bins from b_pub up, where b_pub is the highest bin whose suffix count
//   reaches cmin (one bin higher when that would overflow the list), and u = the largest key
//   below b_pub (0 when none). Nothing else leaves the workgroup: no score array, no global
//   histogram.
// topk (grid: one workgroup of 1024 threads per slot). The workgroup takes the union U of the
//   slot's lists into registers and T = the kk-th largest key of U (1 when U holds fewer than kk
//   keys: then every key counts).
//   U is a subset of all keys, so T is at most the true kk-th largest key. A range whose bound is
//   below T therefore has no unpublished key in the top-kk: its part of the top-kk is in U. A range
//   whose bound is at least T is scored again in full, its list replaced by all its keys >= T,
//   and T recomputed (it can only rise, so the remaining ranges are checked against the new T).
//   The keys >= T that remain are exactly the top-kk. They are bucket-sorted in LDS with bins
//   fitted to their key range; a key's output position is its bin's start plus the number of
//   larger keys in its bin, and idx and score are written from there. With random keys a range holds about kk * range / visible of the top-kk and publishes
//   several times that, so the re-scoring path is rare; it keeps the result exact when the
//   relevant entries cluster (many of the top-kk in one range, or ties).
#include <math.h>

#include "index_common.h"
#include "index_rank.h"

namespace csah {

constexpr int kUMax = 8192;           // union keys a top-k workgroup holds in LDS
constexpr int kCandRange = 4096;      // keys per range at most: the LDS score array
constexpr int kCandMaxRanges = 1024;  // ranges per slot at most (lists of at least 8 keys)
constexpr int kCandThreads = 256;

struct CandWs {
  char* base;
  size_t slot_bytes;
  int R, cap;  // ranges per slot, keys per published list
  __device__ uint64_t* keys(int s) const { return (uint64_t*)(base + (size_t)s * slot_bytes); }
  __device__ uint64_t* bound(int s) const { return keys(s) + (size_t)R * cap; }
};

static inline size_t cand_al256(size_t x) { return (x + 255) & ~(size_t)255; }

// One slot's share of the workspace: every list and bound of the largest plan (R * cap <= kUMax).
size_t index_cand_slot_bytes() { return cand_al256((size_t)(kUMax + kCandMaxRanges) * 8); }

static bool cand_plan_ranges(int64_t n, int64_t chunk, int k, CandPlan* p);

bool index_cand_plan(int slots, int64_t N, int k, int page_shift, CandPlan* p) {
  const int64_t n = N > 0 ? N : 1;
  // about 512 scan workgroups, ranges of 256..4096 keys. Where that would need longer ranges
  // (many keys in all) the ranges shrink towards 2048 keys instead: 16 x 262,144 keys then run as
  // 2048 workgroups, two rounds per CU, so one round's publication overlaps the other's loads
  // (measured 45.8 against 47.6 us; the 4-sequence launch, 512 ranges of 2048, is unchanged)
  int64_t chunk = ((int64_t)slots * n + 511) / 512;
  chunk = (chunk + 255) / 256 * 256;
  if (chunk < 256) chunk = 256;
  if (chunk > kCandRange) {
    chunk = ((int64_t)slots * n + 2047) / 2048;
    chunk = (chunk + 255) / 256 * 256;
    if (chunk < kCandRange / 2) chunk = kCandRange / 2;
    if (chunk > kCandRange) chunk = kCandRange;
  }
  // paged keys: a range spans at most 1024 pages (+1 partial one), which fits the page list
  if (page_shift >= 0 && chunk > ((int64_t)1024 << page_shift)) chunk = (int64_t)1024 << page_shift;
  return cand_plan_ranges(n, chunk, k, p);
}

// Ranges of `chunk` keys over n: R, the list length and the published minimum.
static bool cand_plan_ranges(int64_t n, int64_t chunk, int k, CandPlan* p) {
  const int64_t R = (n + chunk - 1) / chunk;
  if (R > kCandMaxRanges) return false;
  p->chunk = (int)chunk;
  p->R = (int)R;
  int cap = (int)(kUMax / R) & ~7;
  if (cap > chunk) cap = (int)chunk;
  p->cap = cap;
  // a range holds about e of the top-kk; publishing e + 4 sqrt(e) + 8 makes a re-score rare
  const int64_t kk = k < n ? k : n;
  const double e = (double)kk * (double)chunk / (double)n;
  int cmin = (int)ceil(e + 4.0 * sqrt(e) + 8.0);
  if (cmin > cap) cmin = cap;
  if (cmin < 1) cmin = 1;
  p->cmin = cmin;
  return true;
}

// Several queries per sequence: one scan workgroup per (range, sequence) stages every query's
// scores of its range in LDS (Q x (chunk + 4) floats), so the range is capped by that array: 7
// queries of 2048 keys (56 KB; with the histogram and a page list two workgroups still share a CU).
constexpr int kMqStage = 14364;

bool index_cand_plan_mq(int B, int Q, int64_t N, int k, int page_shift, CandPlan* p) {
  if (Q < 1 || Q > kCandMqMaxQ || !index_cand_plan(B, N, k, page_shift, p)) return false;
  const int64_t cmax = (int64_t)((kMqStage / Q - 4) / 256) * 256;
  if (p->chunk <= cmax) return true;
  return cand_plan_ranges(N > 0 ? N : 1, cmax, k, p);
}

// ---- scoring a range ---------------------------------------------------------------------------
// Scores of the keys [g0, g0 + n) of sequence b (1 <= n <= kCandRange) against query slot `slot`
// into stage[0..n); with COUNT also a histogram of the top 12 bits of their order keys. Threads
// 0..255 (four wavefronts) take part; `pages` holds the range's page list when PAGED. The scan
// and the re-scoring in the top-k kernel run this same code, so they produce the same values.

// 128-dim keys, at most 4 indexer heads: v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands takes
// A = 16 keys (lane l: key l%16, 32-element block l/16, with the block's E8M0 scale) and B = the
// query's heads as columns (lane l: head l%16, block l/16; columns past the head count are zero
// codes) and leaves in register i of lane l the head-(l%16) score of key 4(l/16)+i, every product
// exactly scaled. A transposing quad reduction (two exchanges, each sending the values the partner
// keeps) leaves lane c of a quad with key c's sum over the 4 heads. Per head the products are
// exact; while the products' absolute sum spans fewer than 24 bits of the finest granularity every
// partial sum is exact, so the score is the exact one, as in the head-summed form below.
template <bool PAGED, bool COUNT, int U>
__device__ __forceinline__ void score_range_mx(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const EntryMap& kmap, int slot, int b, int64_t g0, int n, const int32_t* pages,
    float* stage, uint32_t* hist) {
  constexpr int STEP = 4 * 16 * U;  // U tiles of 16 keys per wavefront per step, double-buffered
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kb = lane >> 4;
  i32x8 qb = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  int qe = 127;
  if (col < HI) {
    const int64_t qrow = (int64_t)slot * HI + col;
    const u32x4 v = *(const u32x4*)(q_codes + qrow * 64 + 16 * kb);
    qb[0] = (int)v[0];
    qb[1] = (int)v[1];
    qb[2] = (int)v[2];
    qb[3] = (int)v[3];
    qe = q_scales[qrow * 4 + kb];
  }
  const int64_t base_row = PAGED ? 0 : kmap.row(b, g0);
  const uint8_t* kcu = k_codes + base_row * 64;
  const uint8_t* ksu = k_scales + base_row * 4;
  const uint32_t off0 = PAGED ? (uint32_t)(g0 & (((int64_t)1 << kmap.shift) - 1)) : 0u;
  const int wkey = wave * 16 * U + col;  // this lane's key in tile 0 of a step
  auto load = [&](int r0, u32x4* c, uint32_t* e, bool clamp) {
    if (!PAGED && !clamp) {  // workgroup-uniform base per step, per-lane constant offsets
      const uint8_t* pc = kcu + (size_t)(uint32_t)r0 * 64u;
      const uint8_t* ps = ksu + (size_t)(uint32_t)r0 * 4u;
#pragma unroll
      for (int u = 0; u < U; u++) {
        c[u] = __builtin_nontemporal_load(
            (const u32x4*)(pc + (uint32_t)wkey * 64u + 16u * kb + u * 1024));
        e[u] = ps[(uint32_t)wkey * 4u + kb + u * 64];
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      int r = r0 + wkey + 16 * u;
      if (clamp) r = r < n ? r : n - 1;  // rows past the range read a valid row (masked below)
      if constexpr (PAGED) {
        const uint64_t row = page_row(pages, off0 + (uint32_t)r, kmap.shift);
        c[u] = __builtin_nontemporal_load((const u32x4*)(k_codes + row * 64u + 16u * kb));
        e[u] = k_scales[row * 4u + kb];
      } else {
        c[u] = __builtin_nontemporal_load((const u32x4*)(kcu + (uint32_t)r * 64u + 16u * kb));
        e[u] = ksu[(uint32_t)r * 4u + kb];
      }
    }
  };
  const bool hi2 = (col & 2) != 0, hi1 = (col & 1) != 0;
  auto score = [&](int r0, const u32x4* c, const uint32_t* e) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const i32x8 a = i32x8{(int)c[u][0], (int)c[u][1], (int)c[u][2], (int)c[u][3], 0, 0, 0, 0};
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qb, z, 4, 4, 0,
                                                                       (int)e[u], 0, qe);
      // quad lane c: p[j] = head c of key j (of this lane's 4 keys); keep the keys whose bit 1
      // is c's bit 1 and take the partner c^2's heads for them
      const float s0 = (hi2 ? p[2] : p[0]) + quad_read<0x4E>(hi2 ? p[0] : p[2]);
      const float s1 = (hi2 ? p[3] : p[1]) + quad_read<0x4E>(hi2 ? p[1] : p[3]);
      // then key c itself, with the partner c^1's two heads of it
      const float v = (hi1 ? s1 : s0) + quad_read<0xB1>(hi1 ? s0 : s1) + 0.0f;  // -0 -> +0
      const int r = r0 + wave * 16 * U + 16 * u + 4 * kb + col;  // key c = col of the quad
      if (col < 4 && r < n) {
        stage[r] = v;
        if constexpr (COUNT) atomicAdd(&hist[order_key(v) >> kBinShift], 1u);
      }
    }
  };
  u32x4 ca[U], cb[U];
  uint32_t ea[U], eb[U];
  load(0, ca, ea, STEP > n);
  for (int r0 = 0; r0 < n; r0 += 2 * STEP) {
    const bool has_b = r0 + STEP < n;
    if (has_b) load(r0 + STEP, cb, eb, r0 + 2 * STEP > n);
    score(r0, ca, ea);
    if (!has_b) break;
    if (r0 + 2 * STEP < n) load(r0 + 2 * STEP, ca, ea, r0 + 3 * STEP > n);
    score(r0 + STEP, cb, eb);
  }
}

// Other key widths and head counts, on the vector unit. Because the heads are combined by a plain
// sum, the score is one dot product of the key with the head-summed query
// qt_i = sum_h 2^(Eq_h,b(i) - 127) e2m1(q_hi), scaled per key block by 2^(Ek - 127). NB = dI/32
// consecutive lanes score one entry, one 32-element block each; a wavefront takes 64 consecutive
// entries per step and its 16-byte loads cover one contiguous kilobyte of codes.
template <int NB, bool PAGED, bool COUNT, int U>
__device__ __forceinline__ void score_range_valu(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const EntryMap& kmap, int slot, int b, int64_t g0, int n, const int32_t* pages,
    float* stage, uint32_t* hist) {
  constexpr int EPW = 64 / NB;  // entries per wavefront per group of lanes
  constexpr int STEP = 4 * EPW * U;  // U groups whose loads are in flight together
  static_assert(U % NB == 0, "each lane stores U / NB scores");
  const int tid = threadIdx.x, sub = tid % NB;
  // wavefront w takes the entries [w * EPW * U, ...) of each step, group u the EPW entries from
  // u * EPW on (lane q * NB + sub: entry q, block sub)
  const int ent = (tid >> 6) * (EPW * U) + (tid & 63) / NB;
  float qv[32];
#pragma unroll
  for (int j = 0; j < 32; j++) qv[j] = 0.0f;
  for (int h = 0; h < HI; h++) {
    const int64_t qrow = (int64_t)slot * HI + h;
    const u32x4 w = *(const u32x4*)(q_codes + qrow * (16 * NB) + 16 * sub);
    const float s = e8m0_to_f32(q_scales[qrow * NB + sub]);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f32x2 v0 = fp4x2_to_f32<0>(w[j]), v1 = fp4x2_to_f32<1>(w[j]);
      const f32x2 v2 = fp4x2_to_f32<2>(w[j]), v3 = fp4x2_to_f32<3>(w[j]);
      qv[8 * j + 0] += v0[0] * s;
      qv[8 * j + 1] += v0[1] * s;
      qv[8 * j + 2] += v1[0] * s;
      qv[8 * j + 3] += v1[1] * s;
      qv[8 * j + 4] += v2[0] * s;
      qv[8 * j + 5] += v2[1] * s;
      qv[8 * j + 6] += v3[0] * s;
      qv[8 * j + 7] += v3[1] * s;
    }
  }
  const int64_t base_row = PAGED ? 0 : kmap.row(b, g0);
  const uint8_t* kc = k_codes + base_row * (16 * NB) + 16 * sub;
  const uint8_t* ks = k_scales + base_row * NB + sub;
  const uint8_t* kcu = k_codes + base_row * (16 * NB);
  const uint8_t* ksu = k_scales + base_row * NB;
  const uint32_t lane_c = (uint32_t)ent * (16u * NB) + 16u * sub;
  const uint32_t lane_s = (uint32_t)ent * NB + sub;
  const uint32_t off0 = PAGED ? (uint32_t)(g0 & (((int64_t)1 << kmap.shift) - 1)) : 0u;
  auto load = [&](int r0, u32x4* c, uint32_t* e, bool clamp) {
    if (!PAGED && !clamp) {
      const uint8_t* pc = kcu + (size_t)(uint32_t)r0 * (16u * NB);
      const uint8_t* ps = ksu + (size_t)(uint32_t)r0 * NB;
#pragma unroll
      for (int u = 0; u < U; u++) {
        c[u] = __builtin_nontemporal_load((const u32x4*)(pc + lane_c + u * (EPW * 16 * NB)));
        e[u] = ps[lane_s + u * (EPW * NB)];
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      int r = r0 + u * EPW + ent;
      if (clamp) r = r < n ? r : n - 1;
      if constexpr (PAGED) {
        const uint64_t row = page_row(pages, off0 + (uint32_t)r, kmap.shift);
        c[u] = __builtin_nontemporal_load((const u32x4*)(kc + row * (16u * NB)));
        e[u] = ks[row * NB];
      } else {
        c[u] = __builtin_nontemporal_load((const u32x4*)(kc + (uint32_t)r * (16u * NB)));
        e[u] = ks[(uint32_t)r * NB];
      }
    }
  };
  auto score = [&](int r0, const u32x4* c, const uint32_t* e) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; u++) s[u] = block_score<NB>(c[u], e[u], qv);  // in all NB lanes
#pragma unroll
    for (int j = 0; j < U / NB; j++) {
      // lane (q, sub) stores group j * NB + sub's score of its entry q
      float v = s[j * NB];
#pragma unroll
      for (int t = 1; t < NB; t++) v = sub == t ? s[j * NB + t] : v;
      const int r = r0 + (j * NB + sub) * EPW + ent;
      if (r < n) {
        stage[r] = v;
        if constexpr (COUNT) atomicAdd(&hist[order_key(v) >> kBinShift], 1u);
      }
    }
  };
  u32x4 ca[U], cb[U];
  uint32_t ea[U], eb[U];
  load(0, ca, ea, STEP > n);
  for (int r0 = 0; r0 < n; r0 += 2 * STEP) {
    const bool has_b = r0 + STEP < n;
    if (has_b) load(r0 + STEP, cb, eb, r0 + 2 * STEP > n);
    score(r0, ca, ea);
    if (!has_b) break;
    if (r0 + 2 * STEP < n) load(r0 + 2 * STEP, ca, ea, r0 + 3 * STEP > n);
    score(r0 + STEP, cb, eb);
  }
}

// DEEP: four loads per lane in flight (the scan); otherwise as few as the lane layout allows (the
// top-k kernel's re-scoring, which must stay within 128 registers). Each key's arithmetic is the
// same either way.
template <bool MX, int NB, bool PAGED, bool COUNT, bool DEEP>
__device__ __forceinline__ void score_range(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const EntryMap& kmap, int slot, int b, int64_t g0, int n, const int32_t* pages,
    float* stage, uint32_t* hist) {
  if constexpr (MX)
    score_range_mx<PAGED, COUNT, DEEP ? 4 : 1>(q_codes, q_scales, HI, k_codes, k_scales, kmap,
                                                slot, b, g0, n, pages, stage, hist);
  else
    score_range_valu<NB, PAGED, COUNT, DEEP ? 4 : NB>(q_codes, q_scales, HI, k_codes, k_scales,
                                                       kmap, slot, b, g0, n, pages, stage, hist);
}

// The top-k kernel's re-scoring of one range, out of line: it runs rarely, and kept apart its
// registers do not crowd the top-k kernel's own (1024 threads leave 128 per lane).
template <bool MX, int NB, bool PAGED>
__device__ __attribute__((noinline)) void rescore_range(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int slot, int b, int64_t g0, int n, const int32_t* pages, float* stage) {
  score_range<MX, NB, PAGED, false, false>(q_codes, q_scales, HI, k_codes, k_scales, kmap, slot, b,
                                           g0, n, pages, stage, nullptr);
}

__device__ __forceinline__ uint64_t make_key(float s, int64_t g) {
  return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)g);
}
// ---- scan: score a range, publish its list and bound ------------------------------------------
// stage[0..n): the range's scores (entry g0 + j), hist: their 4096-bin histogram. Writes the
// published keys to out[0..cap) (in no particular order: the top-k ranks by value), zero padded,
// and the largest unpublished key (0: none) to *bnd. Three barriers.
__device__ void publish_candidates(const float* stage, const uint32_t* hist, int n, int64_t g0,
                                   int cmin, int cap, uint64_t* __restrict__ out,
                                   uint64_t* __restrict__ bnd) {
  constexpr int NT = kCandThreads, NW = NT / 64, KPT = kCandRange / NT;
  static_assert(kBins == 16 * NT, "each thread owns 16 bins");
  __shared__ uint32_t s_w[NW];
  __shared__ uint32_t s_bpub, s_cnt;
  __shared__ uint64_t s_umax;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) {
    s_bpub = 0;  // publish every bin when the range fits the list
    s_cnt = 0;
    s_umax = 0;
  }
  if (n > cap) {  // uniform: b* = the highest bin whose suffix count reaches cmin
    uint32_t h[16];
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const u32x4 v4 = *(const u32x4*)(hist + 16 * t + j);
      h[j] = v4[0];
      h[j + 1] = v4[1];
      h[j + 2] = v4[2];
      h[j + 3] = v4[3];
    }
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) v += h[j];
    const uint32_t pre = wave_prefix_add(v);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63);
    if (lane == 0) s_w[wave] = wtot;
    __syncthreads();
    uint32_t above = wtot - pre;
#pragma unroll
    for (int w = 0; w < NW; w++) above += w > wave ? s_w[w] : 0u;
    const uint32_t r = (uint32_t)cmin;
    if (above < r && above + v >= r) {  // this thread's bins hold the cmin-th largest
      uint32_t bsel = 16 * t, with_b = 0;
#pragma unroll
      for (int j = 15; j >= 0; j--) {
        if (with_b == 0 && above + h[j] >= r) {
          bsel = 16 * t + j;
          with_b = above + h[j];  // keys in the bins from bsel up
        }
        above += h[j];
      }
      s_bpub = with_b <= (uint32_t)cap ? bsel : bsel + 1;  // the bins above hold < cmin <= cap
    }
  }
  __syncthreads();
  const uint32_t bpub = s_bpub;
  uint64_t umax = 0;
#pragma unroll
  for (int j = 0; j < KPT; j++) {  // item t + 256 j: conflict-free LDS reads
    const int at = t + NT * j;
    if (at >= n) break;
    const float v = stage[at];
    const uint64_t key = make_key(v, g0 + at);
    if ((order_key(v) >> kBinShift) >= bpub) out[atomicAdd(&s_cnt, 1u)] = key;
    else umax = max_u64(umax, key);
  }
  umax = wave_max_u64(umax);
  if (lane == 0 && umax) atomicMax((unsigned long long*)&s_umax, (unsigned long long)umax);
  __syncthreads();
  for (int j = (int)s_cnt + t; j < cap; j += NT) out[j] = 0;
  if (t == 0) *bnd = s_umax;
}

template <bool MX, int NB, bool PAGED>
__global__ __launch_bounds__(kCandThreads) void index_cand_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int chunk, int cmin, CandWs cw) {
  const int slot = blockIdx.y, r = blockIdx.x, b = slot / Q, i = slot - b * Q;
  __shared__ uint32_t hist[kBins];
  __shared__ __attribute__((aligned(16))) float stage[kCandRange];
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  for (int j = threadIdx.x; j < kBins; j += kCandThreads) hist[j] = 0u;
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int64_t g0 = (int64_t)r * chunk;
  const int n = g0 < nv ? (int)(nv - g0 < chunk ? nv - g0 : chunk) : 0;
  if constexpr (PAGED) {
    if (n > 0) load_page_list(kmap, b, g0, g0 + n, pages, threadIdx.x, kCandThreads);
  }
  __syncthreads();
  if (n > 0)
    score_range<MX, NB, PAGED, true, true>(q_codes, q_scales, HI, k_codes, k_scales, kmap, slot, b, g0,
                                     n, pages, stage, hist);
  __syncthreads();
  publish_candidates(stage, hist, n, g0, cmin, cw.cap, cw.keys(slot) + (size_t)r * cw.cap,
                     cw.bound(slot) + r);
}

// ---- top-k over the union ----------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkKPT = kUMax / kTopkThreads;  // union keys per thread, in registers

// One workgroup per slot.
template <bool MX, int NB, bool PAGED>
__global__ __launch_bounds__(kTopkThreads) void index_cand_topk_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int chunk, int k, CandWs cw,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  constexpr int NT = kTopkThreads, KPT = kTopkKPT;
  const int slot = blockIdx.x;
  const int b = slot / Q, i = slot - b * Q, t = threadIdx.x;
  __shared__ __attribute__((aligned(16))) uint64_t buf[kUMax];
  __shared__ uint32_t hist[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t stage_u[kCandRange];
  __shared__ uint64_t bnd[kCandMaxRanges];
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  __shared__ int s_next;
  float* stage = (float*)stage_u;
  const int R = cw.R, nU = R * cw.cap;  // nU <= kUMax
  uint64_t x[KPT];
  {  // the union straight into registers, 16-byte loads all in flight together (which key sits
     // in which register does not matter: the ranking goes by value)
    const u32x4* src = (const u32x4*)cw.keys(slot);
#pragma unroll
    for (int j = 0; j < KPT / 2; j++) {
      const int at = t + NT * j;  // key pair at, nU even
      const u32x4 v = 2 * at < nU ? __builtin_nontemporal_load(src + at) : u32x4{0u, 0u, 0u, 0u};
      x[2 * j] = ((uint64_t)v[1] << 32) | v[0];
      x[2 * j + 1] = ((uint64_t)v[3] << 32) | v[2];
    }
    const uint64_t* bs = cw.bound(slot);
    for (int j = t; j < R; j += NT) bnd[j] = bs[j];
    if (t == 0) s_next = 0x7FFFFFFF;
  }
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const uint32_t kk = (uint32_t)(nv < k ? nv : k);
  int32_t* io = idx_out + (int64_t)slot * k;
  float* so = score_out ? score_out + (int64_t)slot * k : nullptr;
  for (int j = (int)kk + t; j < k; j += NT) {
    io[j] = -1;
    if (so) so[j] = -INFINITY;
  }
  if (kk == 0) return;
  uint64_t T = top_sorted<NT, KPT>(x, kk, hist, stage_u, buf, io, so);
  // a range whose bound reaches T holds unlisted keys that may rank below kk: those ranges are
  // scored again, in index order, and the ranking redone over the result
  for (int w = t; w < R; w += NT)
    if (bnd[w] >= T) atomicMin(&s_next, w);
  __syncthreads();
  int w = s_next;
  __syncthreads();
  if (w >= R) return;
  // every register slot is considered (the union's pair layout is not compact_regs' item order);
  // empty slots hold 0 < T
  int n = compact_regs<NT, KPT>(x, kUMax, [&](uint64_t y) { return y >= T; }, buf, 0);
  for (;;) {
    const int64_t g0 = (int64_t)w * chunk;
    const int gn = (int)(nv - g0 < chunk ? nv - g0 : chunk);  // >= 1: a nonzero bound
    const uint32_t lo = (uint32_t)g0, hi = (uint32_t)(g0 + gn);
    load_regs<NT, KPT>(buf, n, x);
    __syncthreads();
    n = compact_regs<NT, KPT>(x, n, [&](uint64_t y) {
      const uint32_t g = 0xFFFFFFFFu - (uint32_t)y;
      return g < lo || g >= hi;
    }, buf, 0);
    if constexpr (PAGED) {
      load_page_list(kmap, b, g0, g0 + gn, pages, t, NT);
      __syncthreads();
    }
    if (t < kCandThreads)  // the scoring loop takes four wavefronts
      rescore_range<MX, NB, PAGED>(q_codes, q_scales, HI, k_codes, k_scales, kmap, slot, b, g0, gn,
                                   pages, stage);
    __syncthreads();
    {  // append the range's keys >= T (n <= kk <= 4096 before, gn <= 4096 more)
      constexpr int SPT = kCandRange / NT;
      uint64_t y[SPT];
#pragma unroll
      for (int j = 0; j < SPT; j++) {
        const int at = t + NT * j;
        y[j] = at < gn ? make_key(stage[at], g0 + at) : 0;
      }
      n += compact_regs<NT, SPT>(y, gn, [&](uint64_t z) { return z >= T; }, buf, n);
    }
    load_regs<NT, KPT>(buf, n, x);
    __syncthreads();
    T = top_sorted<NT, KPT>(x, kk, hist, stage_u, buf, io, so);
    n = compact_regs<NT, KPT>(x, n, [&](uint64_t y) { return y >= T; }, buf, 0);
    if (t == 0) s_next = 0x7FFFFFFF;
    __syncthreads();
    for (int v = w + 1 + t; v < R; v += NT)
      if (bnd[v] >= T) atomicMin(&s_next, v);
    __syncthreads();
    w = s_next;
    __syncthreads();
    if (w >= R) break;
  }
}

// ---- several queries per sequence: one pass per range for all of them ----------------------------
// The MFMA tiles of the multi-query walk score 16 keys against every query of sequence b (one
// product per indexer head, the heads summed in the accumulator), so the keys are read once for
// all Q queries. Lane n's query is n; its scores of the range go to its row of `stage` (rows
// padded by 4 floats, so that the 16 queries' stores of one key fall in different banks). Then,
// query by query, the row is counted into the 4096-bin histogram and published exactly as the
// one-query scan publishes: a list and a bound for slot b * Q + q in range r. Every score is the
// exact one, so it equals the one-query scoring's value bit for bit (the top-k re-scores a range
// with that code).
template <int HP, bool PAGED>
__global__ __launch_bounds__(kCandThreads) void index_cand_mq_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int chunk, int cmin, CandWs cw) {
  const int r = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  __shared__ __attribute__((aligned(16))) float stage[kMqStage];
  __shared__ uint32_t hist[kBins];
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  const int64_t g0 = (int64_t)r * chunk;
  const int stride = chunk + 4;
  mfma_walk_keys<HP, PAGED>(q_codes, q_scales, HI, k_codes, k_scales, kmap, N, pos, m, Q, b, 0,
                            g0, g0 + chunk, pages, [&](int64_t key, const f32x4& sc, int nvis) {
                              // only lanes of queries below Q get here (the others see no key)
                              float* st = stage + (threadIdx.x & 15) * stride + (int)(key - g0);
                              if (nvis == 4) {
                                *(f32x4*)st = sc;  // key - g0 and the stride are multiples of 4
                              } else {
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                  if (i < nvis) st[i] = sc[i];
                              }
                            });
  for (int q = 0; q < Q; q++) {
    __syncthreads();  // the stage is complete, the previous publication has read the histogram
    for (int j = t; j < kBins; j += kCandThreads) hist[j] = 0u;
    const int64_t nv = visible_entries(pos, b, q, m, N);
    const int n = g0 < nv ? (int)(nv - g0 < chunk ? nv - g0 : chunk) : 0;
    const float* sq = stage + q * stride;
    __syncthreads();
    for (int j = t; j < n; j += kCandThreads) atomicAdd(&hist[order_key(sq[j]) >> kBinShift], 1u);
    __syncthreads();
    const int slot = b * Q + q;
    publish_candidates(sq, hist, n, g0, cmin, cw.cap, cw.keys(slot) + (size_t)r * cw.cap,
                       cw.bound(slot) + r);
  }
}

// ---- launch ------------------------------------------------------------------------------------
template <bool MX, int NB, bool PAGED>
static void launch_cand_t(const IndexArgs& a, const CandPlan& p, const CandWs& w, hipStream_t s) {
  const int slots = a.B * a.Q;
  a.prof.launch(index_cand_scan_kernel<MX, NB, PAGED>, dim3((unsigned)p.R, (unsigned)slots),
                dim3(kCandThreads), s, a.q_codes, a.q_scales, a.HI, a.k_codes, a.k_scales, a.kmap,
                a.N, a.pos, a.m, a.Q, p.chunk, p.cmin, w);
  index_cand_topk_kernel<MX, NB, PAGED><<<dim3((unsigned)slots), kTopkThreads, 0, s>>>(
      a.q_codes, a.q_scales, a.HI, a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, p.chunk,
      a.k, w, a.idx_out, a.score_out);
}

template <bool MX, int NB>
static void launch_cand_p(const IndexArgs& a, const CandPlan& p, const CandWs& w, hipStream_t s) {
  if (a.kmap.table) launch_cand_t<MX, NB, true>(a, p, w, s);
  else launch_cand_t<MX, NB, false>(a, p, w, s);
}

template <int HP, bool PAGED>
static void launch_cand_mq_scan(const IndexArgs& a, const CandPlan& p, const CandWs& w,
                                hipStream_t s) {
  a.prof.launch(index_cand_mq_scan_kernel<HP, PAGED>, dim3((unsigned)p.R, (unsigned)a.B),
                dim3(kCandThreads), s, a.q_codes, a.q_scales, a.HI, a.k_codes, a.k_scales, a.kmap,
                a.N, a.pos, a.m, a.Q, p.chunk, p.cmin, w);
}

template <bool MX, int NB, bool PAGED>
static void launch_cand_topk(const IndexArgs& a, const CandPlan& p, const CandWs& w,
                             hipStream_t s) {
  index_cand_topk_kernel<MX, NB, PAGED><<<dim3((unsigned)(a.B * a.Q)), kTopkThreads, 0, s>>>(
      a.q_codes, a.q_scales, a.HI, a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, p.chunk,
      a.k, w, a.idx_out, a.score_out);
}

hipError_t launch_index_cand_mq(const IndexArgs& a, const CandPlan& p) {
  hipStream_t s = (hipStream_t)a.stream;
  CandWs w;
  w.base = (char*)a.ws;
  w.slot_bytes = index_cand_slot_bytes();
  w.R = p.R;
  w.cap = p.cap;
  const bool paged = a.kmap.table != nullptr;
  if (a.HI <= 4) {
    if (paged) launch_cand_mq_scan<4, true>(a, p, w, s);
    else launch_cand_mq_scan<4, false>(a, p, w, s);
  } else if (a.HI <= 8) {
    if (paged) launch_cand_mq_scan<8, true>(a, p, w, s);
    else launch_cand_mq_scan<8, false>(a, p, w, s);
  } else {
    if (paged) launch_cand_mq_scan<16, true>(a, p, w, s);
    else launch_cand_mq_scan<16, false>(a, p, w, s);
  }
  // the top-k re-scores a range with the one-query code: the MFMA form for at most 4 heads
  if (a.HI <= 4) {
    if (paged) launch_cand_topk<true, 4, true>(a, p, w, s);
    else launch_cand_topk<true, 4, false>(a, p, w, s);
  } else {
    if (paged) launch_cand_topk<false, 4, true>(a, p, w, s);
    else launch_cand_topk<false, 4, false>(a, p, w, s);
  }
  return hipGetLastError();
}

hipError_t launch_index_cand(const IndexArgs& a, const CandPlan& p) {
  hipStream_t s = (hipStream_t)a.stream;
  CandWs w;
  w.base = (char*)a.ws;
  w.slot_bytes = index_cand_slot_bytes();
  w.R = p.R;
  w.cap = p.cap;
  if (a.dI == 128 && a.HI <= 4) launch_cand_p<true, 4>(a, p, w, s);
  else if (a.dI == 32) launch_cand_p<false, 1>(a, p, w, s);
  else if (a.dI == 64) launch_cand_p<false, 2>(a, p, w, s);
  else launch_cand_p<false, 4>(a, p, w, s);
  return hipGetLastError();
}

}  // namespace csah
