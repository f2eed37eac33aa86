// index_topk.hip -- FP4 lightning-indexer scan and exact top-k selection.
//
// [EXPL] "DeepSeek V4 Architecture Explained: CSA, HCA, mHC and Muon", section "How
// compress-then-sparsify attention works": indexer queries are scored against compressed indexer
// keys and each query keeps its top-k entries. [LLMB] "Inside DeepSeek-V4 ...", section
// "1. Compressed Sparse Attention (CSA)": an FP4 indexer computes coarse relevance scores and keeps
// the top 1,024 compressed blocks. [BSWEN] "How DeepSeek V4 Handles 1M Token Context with Hybrid
// Attention", section "Component 3: DeepSeek Sparse Attention (DSA)": score every compressed entry,
// select the top k, attend only to those.
//
// Score of entry g:  sum_h sum_b 2^(Eq_hb+Ek_gb-254) sum_{i in b} e2m1(q_hi) e2m1(k_gi).
// Because the heads are combined by a plain sum, the score is one dot product of the key with the
// head-summed query qt_i = sum_h 2^(Eq_h,b(i)-127) e2m1(q_hi), scaled per key block:
//   score_g = sum_b 2^(Ek_gb-127) sum_{i in b} qt_i e2m1(k_gi).
// Every term is a partial sum of the exact products, so when the products' absolute sum spans
// fewer than 24 bits of the finest granularity each fp32 operation is exact: the result is the
// exact score in any order, and the selection below is bit-exact.
//
// Schedules. Decode calls (one or two queries per sequence) over at most 2^22 entries per
// sequence take the candidate-list scan and top-k of index_cand.hip. A prefill chunk (16 or more
// queries of one sequence, 128-dim keys) takes the sampled-threshold MFMA passes at the end of
// this file, 3 to 15 queries take the multi-query MFMA scan, and everything else takes the
// pipeline below, per (sequence, query) "slot", four kernels. Kernel boundaries carry the
// cross-workgroup dependencies: measured on MI355X, a dependent kernel costs about 1.7 us inside
// a graph, an in-kernel ticket-ordered hand-off about 1.3 us with one workgroup per phase and far
// more with many (same-address atomics serialize, about 8 ns each).
//   prep      qt (fp32, dI values) + clear the histogram / counters        (1 WG per slot)
//   scan      stream the FP4 keys (coalesced 16-byte loads, one 32-element block per lane,
//             8 groups of loads in flight), write fp32 scores, build a 4096-bin histogram of the
//             top 12 bits of each score's order key in LDS, flush it with global atomics; the
//             scores come from the scaled FP4 MFMA per head (128-dim keys, at most 4 heads:
//             index_scan_mx_kernel) or from qt on the vector unit (index_scan_kernel)
//   select    every workgroup finds the bin holding the k-th largest score from the histogram;
//             entries above it ("sure") and in it ("tie") are appended as 64-bit keys
//             (order_key(score) << 32 | ~g, unique per entry) at offsets from a block prefix sum
//             and one atomic per workgroup and list
//   rank      the output position of each candidate is the number of candidates with a greater
//             key (keys are unique; descending key = score descending, index ascending), counted
//             over the candidate's own list (sure or tie) by 16 lanes per group of 4 candidates
//             over many workgroups; when the candidates exceed LDS (massive ties) one workgroup
//             radix-selects the tie list and sorts in LDS
#include "csah_internal.h"
#include "device_common.h"
#include "index_common.h"
#include "index_rank.h"

namespace csah {

// Scan launch shape: workgroups per launch (the key range is split evenly among them) and load
// groups in flight per lane (each double-buffered).
#ifndef CSAH_SCAN_WGS
#define CSAH_SCAN_WGS 512
#endif
#ifndef CSAH_SCAN_U
#define CSAH_SCAN_U 4
#endif
constexpr int kSortCap = 4096;

struct IdxWs {
  char* base;
  size_t slot_bytes, off_hist, off_ctr, off_scores, off_sure, off_tie;
  uint32_t tie_cap;  // keys the tie list holds
  __device__ char* slot(int s) const { return base + (size_t)s * slot_bytes; }
  __device__ float* qt(int s) const { return (float*)slot(s); }
  __device__ uint32_t* hist(int s) const { return (uint32_t*)(slot(s) + off_hist); }
  __device__ uint32_t* ctr(int s) const { return (uint32_t*)(slot(s) + off_ctr); }
  __device__ float* scores(int s) const { return (float*)(slot(s) + off_scores); }
  __device__ uint64_t* sure(int s) const { return (uint64_t*)(slot(s) + off_sure); }
  __device__ uint64_t* tie(int s) const { return (uint64_t*)(slot(s) + off_tie); }
};

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Candidate list of a prefill query (the MFMA path): the keys at or above its sampled threshold
// estimate, about 2.3 kk whatever N is (see index_sample_thresh_kernel); 4 k keys and at least
// twice the LDS ranking's capacity hold them, and a query with more is finished by
// index_rescan_kernel. The list first holds the query's sampled scores (at most kSortCap * 2
// floats). A 4096-query chunk's workspace is then a few hundred MB for any cache length.
static uint32_t prefill_tie_cap(int64_t N, int k) {
  int64_t c = 4 * (int64_t)k;
  if (c < 2 * kSortCap) c = 2 * kSortCap;
  if (c > N) c = N;
  return (uint32_t)c;
}

// Per-slot layout. The scan path stores every score and can take every key as a tie; the MFMA
// path recomputes the scores instead and caps the tie list.
static IdxWs make_ws(void* base, int64_t N, int k, bool with_scores) {
  IdxWs w;
  w.base = (char*)base;
  w.tie_cap = with_scores ? (uint32_t)N : prefill_tie_cap(N, k);
  w.off_hist = al256(128 * sizeof(float));
  w.off_ctr = w.off_hist + al256(kBins * sizeof(uint32_t));
  w.off_scores = w.off_ctr + 256;
  w.off_sure = w.off_scores + (with_scores ? al256((size_t)N * sizeof(float)) : 0);
  w.off_tie = w.off_sure + al256((size_t)k * sizeof(uint64_t));
  w.slot_bytes = w.off_tie + al256((size_t)w.tie_cap * sizeof(uint64_t));
  return w;
}

// Queries of one sequence share its keys; from 16 of them on (one MFMA tile) with 128-dim keys and
// at most 16 indexer heads the scores come from the scaled FP4 MFMA (see index_mfma_select_kernel).
static bool use_mfma_path(int Q, int HI, int dI) { return dI == 128 && Q >= 16 && HI <= 16; }
// From 3 to 15 queries per sequence the scores come from the same MFMA tiles in one pass over the
// keys and are stored, then selected and ranked as in the one-query scan (with 2, scanning the
// keys once per query on the VALU is still faster).
static bool use_mfma_scan(int Q, int HI, int dI) { return dI == 128 && Q >= 3 && Q < 16 && HI <= 16; }

// One or two queries per sequence: the candidate-list schedule of index_cand.hip. Its plan depends on
// the page size only through the range length; up to 2^20 keys every page size fits it, beyond
// that the workspace also covers the stored-score schedule below.
static bool use_cand(int Q, int HI, int dI) { return !use_mfma_path(Q, HI, dI) && !use_mfma_scan(Q, HI, dI); }

size_t index_workspace_bytes(int B, int Q, int64_t N, int k, int HI, int dI) {
  const size_t slots = (size_t)B * (size_t)Q;
  if (use_cand(Q, HI, dI)) {
    const size_t c = slots * index_cand_slot_bytes();
    if (N <= ((int64_t)1 << 20)) return c;
    const size_t o = slots * make_ws(nullptr, N, k, true).slot_bytes;
    return c > o ? c : o;
  }
  IdxWs w = make_ws(nullptr, N, k, !use_mfma_path(Q, HI, dI));
  const size_t o = slots * w.slot_bytes;
  if (use_mfma_scan(Q, HI, dI) && Q <= kCandMqMaxQ) {  // either multi-query schedule may run
    const size_t c = slots * index_cand_slot_bytes();
    return c > o ? c : o;
  }
  return o;
}

// ---- prep: head-summed query and cleared counters ---------------------------------------------
__global__ __launch_bounds__(256) void index_prep_kernel(const uint8_t* __restrict__ q_codes,
                                                          const uint8_t* __restrict__ q_scales,
                                                          int HI, int dI, IdxWs ws) {
  const int slot = blockIdx.x, t = threadIdx.x;
  if (t < dI) {
    float acc = 0.0f;
    for (int h = 0; h < HI; h++) {
      const uint32_t byte = q_codes[((int64_t)slot * HI + h) * (dI / 2) + t / 2];
      const f32x2 v = fp4x2_to_f32<0>(byte);
      const float s = e8m0_to_f32(q_scales[((int64_t)slot * HI + h) * (dI / 32) + t / 32]);
      acc += ((t & 1) ? v[1] : v[0]) * s;
    }
    ws.qt(slot)[t] = acc;
  }
  uint32_t* h = ws.hist(slot);
  for (int j = t; j < kBins; j += 256) h[j] = 0u;
  if (t < 64) ws.ctr(slot)[t] = 0u;
}

// ---- scan --------------------------------------------------------------------------------------
template <int NB, bool PAGED>
__global__ __launch_bounds__(256) void index_scan_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int chunk, IdxWs ws) {
  constexpr int EPW = 64 / NB;   // entries per wavefront per group of lanes
  constexpr int U = CSAH_SCAN_U;  // groups whose loads are in flight together
  constexpr int STEP = 4 * EPW * U;
  static_assert(U % NB == 0, "each lane stores U / NB scores");
  const int slot = blockIdx.y, b = slot / Q, i = slot - b * Q;
  const int tid = threadIdx.x, sub = tid % NB;
  // wavefront w takes the STEP / 4 consecutive entries [w * EPW * U, ...) of each step, group u
  // the EPW entries from u * EPW on (lane q * NB + sub: entry q, block sub), so that after the
  // quad reduction the wavefront writes its U * EPW scores to consecutive words of the LDS stage
  // (U / NB conflict-free writes), from which whole windows go out as 16-byte stores
  const int ent = (tid >> 6) * (EPW * U) + (tid & 63) / NB;
  static_assert(kScoreStage % (2 * STEP) == 0, "a stage window holds whole loop iterations");
  __shared__ uint32_t hist[kBins];
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  __shared__ float stage[kScoreStage];
  for (int j = tid; j < kBins; j += 256) hist[j] = 0u;

  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int64_t g0 = (int64_t)blockIdx.x * chunk;
  const int64_t g1 = g0 + chunk < nv ? g0 + chunk : nv;
  if constexpr (PAGED) {
    if (g0 < nv) load_page_list(kmap, b, g0, g1, pages, tid, 256);
  }
  __syncthreads();
  if (g0 < nv) {
    float qv[32];
    const float* qt = ws.qt(slot) + 32 * sub;
#pragma unroll
    for (int j = 0; j < 32; j++) qv[j] = qt[j];
    // contiguous: per-lane bases, offsets within a chunk fit in 32 bits; paged: bases are the
    // pool and each row goes through the page list (offsets counted from the first page start)
    const int64_t base_row = PAGED ? 0 : kmap.row(b, g0);
    const uint8_t* kc = k_codes + base_row * (16 * NB) + 16 * sub;
    const uint8_t* ks = k_scales + base_row * NB + sub;
    // full steps of contiguous keys: a workgroup-uniform base per step plus a per-lane constant
    // offset, so the loads take no per-step address arithmetic on the vector unit
    const uint8_t* kcu = k_codes + base_row * (16 * NB);
    const uint8_t* ksu = k_scales + base_row * NB;
    const uint32_t lane_c = (uint32_t)ent * (16u * NB) + 16u * sub;
    const uint32_t lane_s = (uint32_t)ent * NB + sub;
    const uint32_t off0 = PAGED ? (uint32_t)(g0 & (((int64_t)1 << kmap.shift) - 1)) : 0u;
    float* sc = ws.scores(slot) + g0;
    const int n = (int)(g1 - g0);
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
          stage[r & (kScoreStage - 1)] = v;
          atomicAdd(&hist[order_key(v) >> kBinShift], 1u);
        }
      }
    };
    // scores [w0, w1) of the stage window go out as coalesced 16-byte stores
    auto flush = [&](int w0, int w1) {
      __syncthreads();
      int j = w0 + 4 * tid;
      for (; j + 4 <= w1; j += 1024)
        *(f32x4*)(sc + j) = *(const f32x4*)(stage + (j & (kScoreStage - 1)));
      for (; j < w1; j++) sc[j] = stage[j & (kScoreStage - 1)];
      __syncthreads();
    };
    // double-buffered groups; full groups need no clamping (control flow is workgroup-uniform)
    u32x4 ca[U], cb[U];
    uint32_t ea[U], eb[U];
    load(0, ca, ea, STEP > n);
    int flushed = 0;
    for (int r0 = 0; r0 < n; r0 += 2 * STEP) {
      const bool has_b = r0 + STEP < n;
      if (has_b) load(r0 + STEP, cb, eb, r0 + 2 * STEP > n);
      score(r0, ca, ea);
      if (!has_b) break;
      if (r0 + 2 * STEP < n) load(r0 + 2 * STEP, ca, ea, r0 + 3 * STEP > n);
      score(r0 + STEP, cb, eb);
      if (((r0 + 2 * STEP) & (kScoreStage - 1)) == 0 && r0 + 2 * STEP < n) {
        flush(flushed, r0 + 2 * STEP);  // a full window, while the next loads are in flight
        flushed = r0 + 2 * STEP;
      }
    }
    flush(flushed, n);
  }
  __syncthreads();
  uint32_t* gh = ws.hist(slot);
  for (int j = tid; j < kBins; j += 256) {
    const uint32_t c = hist[j];
    if (c) atomicAdd(&gh[j], c);
  }
}

// The same scan on the matrix cores, for 128-dim keys and at most 4 indexer heads:
// v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands takes A = 16 keys (lane l: key l%16,
// 32-element block l/16, with the block's E8M0 scale) and B = the query's heads as columns (lane l:
// head l%16, block l/16; columns past the head count are zero codes), and leaves in register i of
// lane l the head-(l%16) score of key 4(l/16)+i, every product exactly scaled. The 4 lanes of a
// quad hold the 4 heads of the same 4 keys; a transposing quad reduction (two exchanges, each
// sending the values the partner keeps) leaves lane c of the quad with key c's sum over the heads.
// That sum is the score of the formula above regrouped (per head instead of head-summed first):
// under the same precondition every partial sum is exact, so it is the same fp32 value. The rest
// (contiguous ranges, LDS score stage, histogram, flushes) is the scan above; a tile of 16 keys
// takes one MFMA and 26 vector instructions instead of about 65 (16 conversions, 32 FMAs and the
// rest per block on the vector path). The kernel stays bound by HBM: taking the arithmetic off the
// vector unit measured 16.7 against 18.4 us at 4 x 262,144 keys and 53.6 against 54.2 at 16.
template <bool PAGED>
__global__ __launch_bounds__(256) void index_scan_mx_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int chunk, IdxWs ws) {
  constexpr int U = CSAH_SCAN_U;  // tiles of 16 keys per wavefront per step
  constexpr int STEP = 4 * 16 * U;
  static_assert(kScoreStage % (2 * STEP) == 0, "a stage window holds whole loop iterations");
  const int slot = blockIdx.y, b = slot / Q, i = slot - b * Q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kb = lane >> 4;  // key of the tile (A) / head (B); 32-element block
  __shared__ uint32_t hist[kBins];
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  __shared__ float stage[kScoreStage];
  for (int j = tid; j < kBins; j += 256) hist[j] = 0u;

  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int64_t g0 = (int64_t)blockIdx.x * chunk;
  const int64_t g1 = g0 + chunk < nv ? g0 + chunk : nv;
  if constexpr (PAGED) {
    if (g0 < nv) load_page_list(kmap, b, g0, g1, pages, tid, 256);
  }
  __syncthreads();
  if (g0 < nv) {
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
    float* sc = ws.scores(slot) + g0;
    const int n = (int)(g1 - g0);
    auto load = [&](int r0, u32x4* c, uint32_t* e, bool clamp) {
      if (!PAGED && !clamp) {  // uniform base per step, per-lane constant offsets
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
        if (clamp) r = r < n ? r : n - 1;
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
          stage[r & (kScoreStage - 1)] = v;
          atomicAdd(&hist[order_key(v) >> kBinShift], 1u);
        }
      }
    };
    auto flush = [&](int w0, int w1) {
      __syncthreads();
      int j = w0 + 4 * tid;
      for (; j + 4 <= w1; j += 1024)
        *(f32x4*)(sc + j) = *(const f32x4*)(stage + (j & (kScoreStage - 1)));
      for (; j < w1; j++) sc[j] = stage[j & (kScoreStage - 1)];
      __syncthreads();
    };
    u32x4 ca[U], cb[U];
    uint32_t ea[U], eb[U];
    load(0, ca, ea, STEP > n);
    int flushed = 0;
    for (int r0 = 0; r0 < n; r0 += 2 * STEP) {
      const bool has_b = r0 + STEP < n;
      if (has_b) load(r0 + STEP, cb, eb, r0 + 2 * STEP > n);
      score(r0, ca, ea);
      if (!has_b) break;
      if (r0 + 2 * STEP < n) load(r0 + 2 * STEP, ca, ea, r0 + 3 * STEP > n);
      score(r0 + STEP, cb, eb);
      if (((r0 + 2 * STEP) & (kScoreStage - 1)) == 0 && r0 + 2 * STEP < n) {
        flush(flushed, r0 + 2 * STEP);
        flushed = r0 + 2 * STEP;
      }
    }
    flush(flushed, n);
  }
  __syncthreads();
  uint32_t* gh = ws.hist(slot);
  for (int j = tid; j < kBins; j += 256) {
    const uint32_t c = hist[j];
    if (c) atomicAdd(&gh[j], c);
  }
}

// Threshold bin of the kk-th largest score from a BINS-bin histogram written by the previous
// kernel (h, suf in LDS): the highest bin whose suffix count reaches kk, and the count above it.
template <int BINS>
__device__ void find_threshold_bin(const uint32_t* __restrict__ gh, int64_t kk, uint32_t* h,
                                   uint32_t* suf, uint32_t* out_bin, uint32_t* out_above) {
  constexpr int PER = BINS / 256;
  __shared__ uint32_t wave_total[4];
  // threads >= 256 only take part in the barriers
  const int t = threadIdx.x, lane = t & 63;
  uint32_t v = 0;
  if (t < 256) {
#pragma unroll
    for (int j = 0; j < PER; j++) {
      const uint32_t c = gh[t * PER + j];
      h[t * PER + j] = c;
      v += c;
    }
  }
  // inclusive suffix sum over the 256 groups: within each wavefront by shuffles, then across the
  // four wavefronts through LDS
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_down((int)v, o, 64);
    if (lane + o < 64) v += y;
  }
  if (t < 256 && lane == 0) wave_total[t >> 6] = v;
  __syncthreads();
  if (t < 256) {
    for (int w = (t >> 6) + 1; w < 4; w++) v += wave_total[w];
    suf[t] = v;
  }
  __syncthreads();
  if (t < 256) {
    const uint32_t mine = suf[t];
    const uint32_t next = t < 255 ? suf[t + 1] : 0u;
    if ((int64_t)mine >= kk && (int64_t)next < kk) {
      uint32_t above = next;
      uint32_t bin = t * PER;
      for (int j = PER - 1; j >= 0; j--) {
        const uint32_t c = h[t * PER + j];
        if ((int64_t)(above + c) >= kk) {
          bin = t * PER + j;
          break;
        }
        above += c;
      }
      *out_bin = bin;
      *out_above = above;
    }
  }
  __syncthreads();
}

// ---- select: candidates above / in the threshold bin, then the exact ordered top-k ----------
__device__ void bitonic_sort_desc(uint64_t* s, int n) {
  // n: power of two; all threads of the block
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
        const int a = 2 * t - (t & (stride - 1));
        const int c = a + stride;
        const uint64_t x = s[a], y = s[c];
        const bool desc = (a & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          s[a] = y;
          s[c] = x;
        }
      }
      __syncthreads();
    }
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelPerThread = 8;
constexpr int kSelChunk = kSelThreads * kSelPerThread;

// bin_bits: width of the histogram bin (top bits of the order key) shared by every tie candidate.
// The candidates (at most kSortCap) are ordered by a bucket ranking in LDS when cnt and cur
// (kBins-entry LDS arrays) are given, else by a bitonic sort.
template <int NT>
__device__ void finalize_slot(int slot, int64_t N, int k, int kk, int32_t* __restrict__ idx_out,
                              float* __restrict__ score_out, IdxWs ws, uint64_t* keys,
                              uint32_t* dh, int bin_bits, uint32_t* cnt = nullptr,
                              uint32_t* cur = nullptr) {
  __shared__ uint64_t s_prefix, s_pmask;
  __shared__ uint32_t s_r, s_cnt;
  const int t = threadIdx.x;
  int32_t* io = idx_out + (int64_t)slot * k;
  float* so = score_out ? score_out + (int64_t)slot * k : nullptr;
  if (kk == 0) {
    for (int j = t; j < k; j += blockDim.x) {
      io[j] = -1;
      if (so) so[j] = -INFINITY;
    }
    return;
  }
  uint32_t* ctr = ws.ctr(slot);
  uint32_t ns = ctr[0], nt = ctr[1];
  ns = ns > (uint32_t)kk ? (uint32_t)kk : ns;
  nt = (int64_t)nt > N ? (uint32_t)N : nt;
  const uint64_t* sure = ws.sure(slot);
  const uint64_t* tie = ws.tie(slot);
  int n;
  if (ns + nt <= (uint32_t)kSortCap) {
    n = (int)(ns + nt);
    for (int j = t; j < n; j += blockDim.x) keys[j] = j < (int)ns ? sure[j] : tie[j - ns];
  } else {
    // radix select the r-th largest tie key (keys are unique), 8 bits at a time below the bin
    const int kLowBits = 64 - bin_bits;  // key bits below the shared bin
    if (t == 0) {
      s_r = (uint32_t)kk - ns;
      s_prefix = 0;
      s_pmask = 0;
    }
    __syncthreads();
    for (int hi = kLowBits; hi > 0;) {
      const int width = hi >= 8 ? 8 : hi;
      const int shift = hi - width;
      const uint64_t dmask = ((uint64_t)1 << width) - 1;
      for (int j = t; j < 256; j += blockDim.x) dh[j] = 0;
      __syncthreads();
      const uint64_t pm = s_pmask, pv = s_prefix;
      for (uint32_t j = t; j < nt; j += blockDim.x) {
        const uint64_t x = tie[j];
        if ((x & pm) == pv) atomicAdd(&dh[(x >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (t == 0) {
        uint32_t r = s_r, cum = 0;
        int d = (int)dmask;
        for (; d > 0; d--) {
          if (cum + dh[d] >= r) break;
          cum += dh[d];
        }
        s_r = r - cum;
        s_prefix = pv | ((uint64_t)d << shift);
        s_pmask = pm | (dmask << shift);
      }
      __syncthreads();
      hi = shift;
    }
    // bits above kLowBits are the (shared) bin: compare the low bits only
    const uint64_t low = kLowBits >= 64 ? ~(uint64_t)0 : ((uint64_t)1 << kLowBits) - 1;
    const uint64_t thr = s_prefix;
    if (t == 0) s_cnt = 0;
    __syncthreads();
    for (int j = t; j < (int)ns; j += blockDim.x) keys[j] = sure[j];
    for (uint32_t j = t; j < nt; j += blockDim.x) {
      const uint64_t x = tie[j];
      if ((x & low) >= thr) {
        const uint32_t at = atomicAdd(&s_cnt, 1u);
        if (ns + at < (uint32_t)kSortCap) keys[ns + at] = x;
      }
    }
    __syncthreads();
    n = (int)(ns + (s_cnt < (uint32_t)kSortCap - ns ? s_cnt : (uint32_t)kSortCap - ns));
  }
  if (cnt) {
    // keys are unique: rank them from the top through buckets fitted to their range (a key's
    // position is its bucket's start plus the larger keys in its bucket) and write the first kk
    constexpr int KPT = kSortCap / NT;
    __syncthreads();
    uint64_t x[KPT];
    load_regs<NT, KPT>(keys, n, x);
    __syncthreads();  // keys now serves as the ranked array
    const int kw = n < kk ? n : kk;
    for (int j = kw + t; j < k; j += NT) {
      io[j] = -1;
      if (so) so[j] = -INFINITY;
    }
    top_sorted<NT, KPT>(x, (uint32_t)kw, cnt, cur, keys, io, so);
    return;
  }
  int p2 = 2;
  while (p2 < n) p2 <<= 1;
  for (int j = n + t; j < p2; j += blockDim.x) keys[j] = 0;
  __syncthreads();
  bitonic_sort_desc(keys, p2);
  for (int j = t; j < k; j += blockDim.x) {
    if (j < kk && j < n) {
      const uint64_t x = keys[j];
      io[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)x);
      if (so) so[j] = key_to_float((uint32_t)(x >> 32));
    } else {
      io[j] = -1;
      if (so) so[j] = -INFINITY;
    }
  }
}

// BINS / SHIFT: the histogram the scan wrote (the top log2(BINS) bits of the order key)
template <int BINS, int SHIFT>
__global__ __launch_bounds__(kSelThreads) void index_select_kernel(
    const int64_t* __restrict__ pos, int m, int Q, int64_t N, int k, IdxWs ws) {
  const int slot = blockIdx.y, b = slot / Q, i = slot - b * Q;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int kk = (int)(nv < k ? nv : k);
  if (kk == 0 || (int64_t)blockIdx.x * kSelChunk >= nv) return;
  __shared__ uint32_t h[BINS];
  __shared__ uint32_t suf[256];
  __shared__ uint32_t s_bin, s_above;
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t s_base[2];
  uint32_t* ctr = ws.ctr(slot);
  const int64_t g0 = (int64_t)blockIdx.x * kSelChunk + (int64_t)t * kSelPerThread;
  const float* sc = ws.scores(slot);
  float v[kSelPerThread];
  if (g0 + kSelPerThread <= nv) {
    const f32x4 a = *(const f32x4*)(sc + g0), c = *(const f32x4*)(sc + g0 + 4);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = c[0]; v[5] = c[1]; v[6] = c[2]; v[7] = c[3];
  } else {
#pragma unroll
    for (int e = 0; e < kSelPerThread; e++) v[e] = g0 + e < nv ? sc[g0 + e] : -INFINITY;
  }
  find_threshold_bin<BINS>(ws.hist(slot), kk, h, suf, &s_bin, &s_above);
  const uint32_t bstar = s_bin;
  uint32_t cls[kSelPerThread];  // 0 drop, 1 sure, 2 tie
  uint32_t cnt = 0;             // sure count | tie count << 16
#pragma unroll
  for (int e = 0; e < kSelPerThread; e++) {
    const uint32_t bin = order_key(v[e]) >> SHIFT;
    cls[e] = (g0 + e < nv) ? (bin > bstar ? 1u : (bin == bstar ? 2u : 0u)) : 0u;
    cnt += cls[e] == 1u ? 1u : (cls[e] == 2u ? 0x10000u : 0u);
  }
  // block-wide exclusive prefix of (sure, tie) counts; one atomic per list per workgroup
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (t == 0) {
    uint32_t tot = 0;
    for (int w = 0; w < kSelThreads / 64; w++) {
      const uint32_t x = wsum[w];
      wsum[w] = tot;
      tot += x;
    }
    s_base[0] = (tot & 0xFFFFu) ? atomicAdd(&ctr[0], tot & 0xFFFFu) : 0u;
    s_base[1] = (tot >> 16) ? atomicAdd(&ctr[1], tot >> 16) : 0u;
  }
  __syncthreads();
  const uint32_t excl = wsum[wave] + incl - cnt;
  uint32_t ps = s_base[0] + (excl & 0xFFFFu), pt = s_base[1] + (excl >> 16);
  uint64_t* sure = ws.sure(slot);
  uint64_t* tie = ws.tie(slot);
#pragma unroll
  for (int e = 0; e < kSelPerThread; e++) {
    const uint64_t key = ((uint64_t)order_key(v[e]) << 32) |
                         (uint64_t)(0xFFFFFFFFu - (uint32_t)(g0 + e));
    if (cls[e] == 1u) {
      if (ps < (uint32_t)k) sure[ps] = key;
      ps++;
    } else if (cls[e] == 2u) {
      if ((int64_t)pt < N) tie[pt] = key;
      pt++;
    }
  }
}

// Ordered top-k by rank counting: keys are unique, so the output position of candidate x is the
// number of candidates greater than x. Every "sure" key lies in a higher histogram bin than every
// "tie" key, so a group of candidates that are all sure counts over the sure keys only, and one
// whose candidates are all tie counts over the tie keys and adds the sure count (counting over
// both lists is right for either kind). A workgroup ranks 64 candidates and stages only the
// list(s) they need in LDS. A group of kRankLanes lanes holds kRankCand consecutive candidates in
// registers, splits the list kRankLanes ways, compares each key it reads with all of them (several
// reads in flight per lane) and sums the partial counts with lane shuffles. Massive ties (more
// candidates than kSortCap) fall back to finalize_slot in workgroup 0.
constexpr int kRankThreads = 256;
constexpr int kRankLanes = 16;
constexpr int kRankCand = 4;
constexpr int kRankPerWG = kRankThreads / kRankLanes * kRankCand;
static_assert(kRankCand == 4 && kSortCap < (1 << 16), "two 16-bit counts per shuffled word");
constexpr int kRankStage = 8;  // staged keys in flight per thread

__global__ __launch_bounds__(kRankThreads) void index_rank_kernel(
    const int64_t* __restrict__ pos, int m, int Q, int64_t N, int k,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out, IdxWs ws, int bin_bits) {
  const int slot = blockIdx.y, b = slot / Q, i = slot - b * Q;
  const int t = threadIdx.x;
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int kk = (int)(nv < k ? nv : k);
  __shared__ uint64_t keys[kSortCap];
  __shared__ uint32_t dh[256];
  const uint32_t* ctr = ws.ctr(slot);
  uint32_t ns = 0, nt = 0;
  if (kk > 0) {
    ns = ctr[0];
    nt = ctr[1];
    ns = ns > (uint32_t)kk ? (uint32_t)kk : ns;
    nt = (int64_t)nt > N ? (uint32_t)N : nt;
  }
  const uint32_t n = ns + nt;
  if (kk == 0 || n > (uint32_t)kSortCap) {
    if (blockIdx.x == 0)
      finalize_slot<kRankThreads>(slot, N, k, kk, idx_out, score_out, ws, keys, dh, bin_bits);
    return;
  }
  int32_t* io = idx_out + (int64_t)slot * k;
  float* so = score_out ? score_out + (int64_t)slot * k : nullptr;
  if (blockIdx.x == 0)
    for (int j = kk + t; j < k; j += kRankThreads) {
      io[j] = -1;
      if (so) so[j] = -INFINITY;
    }
  const uint32_t e0 = (uint32_t)blockIdx.x * kRankPerWG;  // the workgroup ranks [e0, e0 + 64)
  if (e0 >= n) return;
  const uint64_t* sure = ws.sure(slot);
  const uint64_t* tie = ws.tie(slot);
  const uint32_t s0 = e0 < ns ? 0u : ns;                          // staged: [s0, s1)
  const uint32_t s1 = e0 + kRankPerWG <= ns ? ns : n;
  for (uint32_t j0 = s0 + t; j0 < s1; j0 += kRankStage * kRankThreads) {  // loads go out together
    uint64_t v[kRankStage];
#pragma unroll
    for (int u = 0; u < kRankStage; u++) {
      const uint32_t j = j0 + u * kRankThreads;
      if (j < s1) v[u] = j < ns ? sure[j] : tie[j - ns];
    }
#pragma unroll
    for (int u = 0; u < kRankStage; u++) {
      const uint32_t j = j0 + u * kRankThreads;
      if (j < s1) keys[j] = v[u];
    }
  }
  __syncthreads();
  const int part = t % kRankLanes;
  const uint32_t c0 = e0 + (uint32_t)(t / kRankLanes) * kRankCand;  // candidates c0 .. c0 + 3
  uint64_t x[kRankCand];
#pragma unroll
  for (int c = 0; c < kRankCand; c++) x[c] = c0 + c < n ? keys[c0 + c] : ~(uint64_t)0;
  // counted range [lo, hi): inside the staged range for every valid candidate of the group
  uint32_t lo = 0, hi = 0;
  if (c0 < n) {
    const uint32_t clast = (c0 + kRankCand < n ? c0 + kRankCand : n) - 1;
    lo = c0 >= ns ? ns : 0u;
    hi = clast < ns ? ns : n;
  }
  uint32_t a[kRankCand] = {};
  uint32_t j = lo + part;
  for (; j + 3 * kRankLanes < hi; j += 4 * kRankLanes) {
    const uint64_t y0 = keys[j], y1 = keys[j + kRankLanes], y2 = keys[j + 2 * kRankLanes],
                   y3 = keys[j + 3 * kRankLanes];
#pragma unroll
    for (int c = 0; c < kRankCand; c++)
      a[c] += (uint32_t)(y0 > x[c]) + (uint32_t)(y1 > x[c]) + (uint32_t)(y2 > x[c]) +
              (uint32_t)(y3 > x[c]);
  }
  for (; j < hi; j += kRankLanes) {
    const uint64_t y = keys[j];
#pragma unroll
    for (int c = 0; c < kRankCand; c++) a[c] += (uint32_t)(y > x[c]);
  }
  // counts stay below 2^16 (n <= kSortCap): two per word through the shuffles
  uint32_t p01 = a[0] | a[1] << 16, p23 = a[2] | a[3] << 16;
#pragma unroll
  for (int o = 1; o < kRankLanes; o <<= 1) {
    p01 += (uint32_t)__shfl_xor((int)p01, o, 64);
    p23 += (uint32_t)__shfl_xor((int)p23, o, 64);
  }
  if (part < kRankCand) {  // lane `part` of the group writes candidate c0 + part
    const uint32_t e = c0 + (uint32_t)part;
    const uint32_t w = part < 2 ? p01 : p23;
    const uint32_t above = ((part & 1) ? w >> 16 : w & 0xFFFFu) + lo;
    const uint64_t xe = part == 0 ? x[0] : part == 1 ? x[1] : part == 2 ? x[2] : x[3];
    if (e < n && above < (uint32_t)kk) {
      io[above] = (int32_t)(0xFFFFFFFFu - (uint32_t)xe);
      if (so) so[above] = key_to_float((uint32_t)(xe >> 32));
    }
  }
}

// ================================================================================================
// Many queries per sequence (prefill chunks): scores on the scaled FP4 MFMA.
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands (format code 4) multiplies a 16 x 128 block
// of FP4 codes by a 128 x 16 block; lane l supplies one 32-element block (16 bytes, the low four
// dwords of the operand) of row l%16, block l/16, with that block's E8M0 scale, and the exactly
// scaled products are accumulated in fp32. With A = 16 keys and B = 16 queries of one indexer head,
// one instruction per head into the same accumulator leaves score(key 4*(l/16)+i, query l%16) in
// register i of lane l. Every product is exact, so under the same precondition as the scan (the
// absolute sum spans fewer than 24 bits of the finest granularity) the scores are the exact ones in
// any accumulation order, and every pass below computes bit-identical values.
//   clear    zero the per-query counters
//   sample   score kSampleSegs segments of kSampleSeg keys spread over each query block's keys
//   thresh   per query: an exact order statistic of its sampled scores as the threshold estimate
//   select   the one full pass: keys at or above the estimate appended to the query's list
//   sort     per query: the list ranked in LDS (after a radix select when it exceeds kSortCap),
//            then the ordered top-k
//   rescan   per query whose list holds fewer than kk keys or more than its capacity: an exact
//            radix select over fresh passes across its keys, then the ranking
constexpr int kPBins = 2048, kPBinShift = 21;
constexpr int kPKeys = 16384;                // keys per workgroup: a 16-bit counter cannot overflow
constexpr uint32_t kNoThreshold = 0xFFFFFFFFu;

// Work split: the keys are cut into nkr ranges (a multiple of 8, at most kPKeys keys each) and the
// queries into blocks of 16. Workgroups are dispatched round-robin over the 8 XCDs (id % 8), so
// XCD x takes the key ranges x, x+8, ... for every query block: its few ranges stay resident in
// its own L2 while all query blocks stream over them.
struct MfmaSplit {
  int nkr, nqb, B;  // grid = nkr * nqb * B workgroups (a multiple of 8)
  int64_t keys_per_range;
};

__device__ __forceinline__ void mfma_unit(const MfmaSplit& sp, int& b, int& qb, int& kr) {
  const int w = blockIdx.x, xcd = w & 7, i = w >> 3;
  const int per = sp.nkr >> 3;  // key ranges per XCD
  const int kl = i % per, rest = i / per;
  kr = xcd + 8 * kl;
  qb = rest % sp.nqb;
  b = rest / sp.nqb;
}

// Key range kr of the split.
template <int HP, bool PAGED, typename F>
__device__ __forceinline__ void mfma_walk(const uint8_t* __restrict__ q_codes,
                                          const uint8_t* __restrict__ q_scales, int HI,
                                          const uint8_t* __restrict__ k_codes,
                                          const uint8_t* __restrict__ k_scales,
                                          const EntryMap& kmap, int64_t N,
                                          const int64_t* __restrict__ pos, int m, int Q,
                                          const MfmaSplit& sp, int b, int qb, int kr,
                                          int32_t* pages, F visit) {
  const int64_t g0 = (int64_t)kr * sp.keys_per_range;
  mfma_walk_keys<HP, PAGED>(q_codes, q_scales, HI, k_codes, k_scales, kmap, N, pos, m, Q, b, qb,
                            g0, g0 + sp.keys_per_range, pages, visit);
}

__global__ __launch_bounds__(256) void index_clear_kernel(IdxWs ws) {
  if (threadIdx.x < 64) ws.ctr(blockIdx.x)[threadIdx.x] = 0u;
}

// ---- prefill: a sampled threshold, one pass, an exact finish ---------------------------------
// kSampleSegs segments of kSampleSeg keys spread evenly over the keys every query of a block sees
// (all of them, contiguous, when those are at most kSampleSegs * kSampleSeg): their scores give
// each query an estimate of its top-k threshold.
constexpr int kSampleSegs = 64, kSampleSeg = 128, kSampleMax = kSampleSegs * kSampleSeg;

__device__ __forceinline__ int64_t sample_seg_start(int64_t nvmin, int s) {
  return nvmin <= kSampleMax ? (int64_t)s * kSampleSeg : (int64_t)s * (nvmin / kSampleSegs);
}
__device__ __forceinline__ int sample_count(int64_t nvmin) {
  return nvmin <= kSampleMax ? (int)nvmin : kSampleMax;
}

// One workgroup per (sequence, block of 16 queries, group of kSampleTilesPerWG tiles of 16 sampled
// keys): the sampled keys' scores of each query go to the start of its tie list (sample position
// p = segment * kSampleSeg + offset), which the select pass later overwrites with candidates. A
// tile lies inside one segment (kSampleSeg is a multiple of 16), and each wavefront loads all its
// tiles at once.
constexpr int kSampleTilesPerWG = 32, kSampleWaveTiles = kSampleTilesPerWG / 4;
constexpr int kSampleGroups = kSampleMax / 16 / kSampleTilesPerWG;

template <int HP, bool PAGED>
__global__ __launch_bounds__(256) void index_mfma_sample_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int nqb, IdxWs ws) {
  const int grp = blockIdx.x % kSampleGroups, rest = blockIdx.x / kSampleGroups;
  const int qb = rest % nqb, b = rest / nqb, q0 = qb * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, blk = lane >> 4;
  // the block's first query sees the fewest keys: the sample lies below that
  const int64_t nvmin = visible_entries(pos, b, q0, m, N);
  const int S = sample_count(nvmin);
  const int ntile = (S + 15) / 16;
  const int t0 = grp * kSampleTilesPerWG + wave;  // this wavefront's tiles: t0 + 4 u
  if (t0 >= ntile) return;                        // per wavefront: no barriers below
  const int qi = q0 + n;
  const bool qv = qi < Q;
  QueryOps<HP> qo;
  load_query_ops<HP>(q_codes, q_scales, HI, (int64_t)b * Q + qi, qv, blk, qo);
  u32x4 c[kSampleWaveTiles];
  uint32_t e[kSampleWaveTiles];
#pragma unroll
  for (int u = 0; u < kSampleWaveTiles; u++) {
    int p = 16 * (t0 + 4 * u) + n;  // sample position of this lane's key in the A operand
    p = p < S ? p : S - 1;          // past the sample: a valid key, scored and dropped
    const int64_t key = sample_seg_start(nvmin, p / kSampleSeg) + p % kSampleSeg;
    const int64_t row = kmap.row(b, key);
    c[u] = __builtin_nontemporal_load((const u32x4*)(k_codes + row * 64 + 16 * blk));
    e[u] = k_scales[row * 4 + blk];
  }
  float* samp = (float*)ws.tie((int)((int64_t)b * Q + (qv ? qi : Q - 1)));
#pragma unroll
  for (int u = 0; u < kSampleWaveTiles; u++) {
    const int tile = t0 + 4 * u;
    if (tile >= ntile) break;  // uniform over the wavefront
    f32x4 sc = tile_scores<HP>(c[u], e[u], qo);
    const int p0 = 16 * tile + 4 * blk;  // positions of this lane's four scores
    if (!qv) continue;
    if (p0 + 4 <= S) {
      *(f32x4*)(samp + p0) = sc;
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (p0 + i < S) samp[p0 + i] = sc[i];
    }
  }
}

// Per query: the threshold estimate, an order key, in ctr[2]. With mu = kk S / nv the expected
// number of the S sampled keys among the true top kk, the estimate is (at most) the m-th largest
// sampled key for m = mu + 6 sqrt(mu) + 8: it lies above the true kk-th largest key only when m or
// more sampled keys do, far in the tail of their distribution, and the keys at or above it then
// number about kk m / mu, a few kk. Queries that see at most kSortCap keys take every key
// (estimate 0). A wrong estimate costs time only: the select pass counts the keys at or above it,
// and a query with fewer than kk or more than its list holds is finished by index_rescan_kernel.
// One wavefront per query, no barriers: where mu exceeds kEstMu only every r-th sampled key is
// used (mu / r at most kEstMu, so m stays below 4 * 64); each lane keeps the 4 largest of its keys,
// and the estimate is the m-th largest of those 256. They are sampled keys, so that value is at
// most the m-th largest sampled key: the estimate can only come out lower, which keeps it safe.
constexpr int kEstMu = 100, kEstKeep = 4;

__global__ __launch_bounds__(256) void index_sample_thresh_kernel(const int64_t* __restrict__ pos,
                                                                  int m, int Q, int64_t N, int k,
                                                                  int slots, IdxWs ws) {
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slot >= slots) return;  // per wavefront: this kernel has no barriers
  const int b = slot / Q, i = slot - b * Q;
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int64_t kk = nv < k ? nv : k;
  uint32_t* ctr = ws.ctr(slot);
  if (kk == 0 || nv <= kSortCap) {
    if (lane == 0) ctr[2] = kk == 0 ? kNoThreshold : 0u;
    return;
  }
  const int S = sample_count(visible_entries(pos, b, i - i % 16, m, N));
  const double mu0 = (double)kk * (double)S / (double)nv;
  const int r = mu0 > kEstMu ? (int)ceil(mu0 / kEstMu) : 1;  // use sampled keys 0, r, 2r, ...
  const int S2 = (S + r - 1) / r;
  const double mu = (double)kk * (double)S2 / (double)nv;
  const int mt = (int)ceil(mu + 6.0 * sqrt(mu) + 8.0);
  if (mt >= S2 || mt > kEstKeep * 64) {  // the sample cannot bound it: take every key
    if (lane == 0) ctr[2] = 0u;
    return;
  }
  const float* samp = (const float*)ws.tie(slot);
  uint32_t top[kEstKeep] = {0u, 0u, 0u, 0u};  // descending; 0: none
  for (int q = lane; q < S2; q += 64) {
    uint32_t x = order_key(samp[(size_t)q * r] + 0.0f);
#pragma unroll
    for (int j = 0; j < kEstKeep; j++) {  // insertion: x moves down past the smaller keys
      const uint32_t hi = x > top[j] ? x : top[j], lo = x > top[j] ? top[j] : x;
      top[j] = hi;
      x = lo;
    }
  }
  // the mt-th largest of the 256 kept keys, one bit at a time from the top
  uint32_t prefix = 0u, rr = (uint32_t)mt;
  for (int bit = 31; bit >= 0; bit--) {
    const uint32_t sel = ~0u << bit, want = prefix | (1u << bit);
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kEstKeep; j++) c += (top[j] != 0u && (top[j] & sel) == want) ? 1u : 0u;
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_add(c), 63);
    if (total >= rr) prefix = want;
    else rr -= total;
  }
  if (lane == 0) ctr[2] = prefix;
}

// The one full pass: every key whose score reaches the query's estimate goes to its candidate
// list (the tie list; ctr[1] counts past the list's end). Candidates are staged per query in LDS
// and appended with one atomic per query and workgroup; a full stage spills straight to the list.
constexpr int kPStage = 256;

template <int HP, bool PAGED>
__global__ __launch_bounds__(256) void index_mfma_select_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, MfmaSplit sp, IdxWs ws) {
  __shared__ uint64_t stage[16][kPStage];
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  __shared__ uint32_t scount[16], sbase[16];
  int b, qb, kr;
  mfma_unit(sp, b, qb, kr);
  const int q0 = qb * 16, n = threadIdx.x & 15;
  if (threadIdx.x < 16) scount[threadIdx.x] = 0u;
  __syncthreads();
  const int qi = q0 + n;
  const int64_t slot = (int64_t)b * Q + (qi < Q ? qi : Q - 1);
  uint32_t* ctr = ws.ctr((int)slot);
  const uint32_t est = qi < Q ? ctr[2] : kNoThreshold;
  // scores below the estimate are dropped with one compare (estimate 0: every key)
  const float smin = est == kNoThreshold ? INFINITY : (est == 0u ? -INFINITY : key_to_float(est));
  uint64_t* cand = ws.tie((int)slot);
  mfma_walk<HP, PAGED>(q_codes, q_scales, HI, k_codes, k_scales, kmap, N, pos, m, Q, sp, b, qb,
                       kr, pages, [&](int64_t key0, const f32x4& sc, int nvis) {
#pragma unroll
                         for (int i = 0; i < 4; i++) {
                           if (i >= nvis) break;
                           const float s = sc[i];
                           if (!(s >= smin)) continue;
                           const uint64_t x = ((uint64_t)order_key(s) << 32) |
                                              (uint64_t)(0xFFFFFFFFu - (uint32_t)(key0 + i));
                           const uint32_t at = atomicAdd(&scount[n], 1u);
                           if (at < (uint32_t)kPStage) {
                             stage[n][at] = x;
                           } else {
                             const uint32_t g = atomicAdd(&ctr[1], 1u);  // counts past the cap
                             if (g < ws.tie_cap) cand[g] = x;
                           }
                         }
                       });
  __syncthreads();
  if (threadIdx.x < 16) {
    const int qn = threadIdx.x;
    const uint32_t c = scount[qn];
    const uint32_t staged = c < (uint32_t)kPStage ? c : (uint32_t)kPStage;
    sbase[qn] = (staged && q0 + qn < Q)
                    ? atomicAdd(&ws.ctr((int)((int64_t)b * Q + q0 + qn))[1], staged)
                    : 0u;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < 16 * kPStage; j += 256) {
    const int qn = j / kPStage, e = j % kPStage;
    const uint32_t c = scount[qn];
    if ((uint32_t)e >= (c < (uint32_t)kPStage ? c : (uint32_t)kPStage) || q0 + qn >= Q) continue;
    const uint32_t g = sbase[qn] + e;
    if (g < ws.tie_cap) ws.tie((int)((int64_t)b * Q + q0 + qn))[g] = stage[qn][e];
  }
}

// A few queries per sequence (multi-token decode): one pass over the keys. The MFMA tiles give
// the scores of all the workgroup's queries at once; each is stored and counted in the query's
// 2048-bin histogram, and index_select_kernel / index_rank_kernel finish as in the one-query scan.
template <int HP, bool PAGED>
__global__ __launch_bounds__(256, 2) void index_mfma_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, MfmaSplit sp, IdxWs ws) {
  __shared__ uint32_t hist[16 * kPBins / 2];  // two 16-bit counters per word
  __shared__ int32_t pages[PAGED ? kPageList : 1];
  int b, qb, kr;
  mfma_unit(sp, b, qb, kr);
  const int n = threadIdx.x & 15, q0 = qb * 16;
  const int words = (Q - q0 < 16 ? Q - q0 : 16) * (kPBins / 2);  // the block's queries only
  for (int j = threadIdx.x; j < words; j += 256) hist[j] = 0u;
  __syncthreads();
  uint32_t* hq = hist + n * (kPBins / 2);
  // lanes of queries past Q visit nothing; point them at a valid slot all the same
  float* sc = ws.scores((int)((int64_t)b * Q + (q0 + n < Q ? q0 + n : Q - 1)));
  mfma_walk<HP, PAGED>(q_codes, q_scales, HI, k_codes, k_scales, kmap, N, pos, m, Q, sp, b, qb,
                       kr, pages, [&](int64_t key0, const f32x4& s4, int nvis) {
                         if (nvis == 4) {
                           *(f32x4*)(sc + key0) = s4;  // key0 is a multiple of 4
                         } else {
#pragma unroll
                           for (int i = 0; i < 4; i++)
                             if (i < nvis) sc[key0 + i] = s4[i];
                         }
#pragma unroll
                         for (int i = 0; i < 4; i++) {
                           if (i >= nvis) break;
                           const uint32_t bin = order_key(s4[i]) >> kPBinShift;
                           atomicAdd(&hq[bin >> 1], 1u << (16 * (bin & 1)));
                         }
                       });
  __syncthreads();
  for (int j = threadIdx.x; j < words; j += 256) {
    const int qn = j / (kPBins / 2), wd = j - qn * (kPBins / 2);
    const uint32_t v = hist[j];
    if (v == 0u || q0 + qn >= Q) continue;
    uint32_t* gh = ws.hist((int)((int64_t)b * Q + q0 + qn));
    if (v & 0xFFFFu) atomicAdd(&gh[2 * wd], v & 0xFFFFu);
    if (v >> 16) atomicAdd(&gh[2 * wd + 1], v >> 16);
  }
}

__global__ __launch_bounds__(1024) void index_sort_kernel(const int64_t* __restrict__ pos, int m,
                                                          int Q, int64_t N, int k,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ score_out,
                                                          IdxWs ws, int bin_bits) {
  const int slot = blockIdx.x, b = slot / Q, i = slot - b * Q;
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int kk = (int)(nv < k ? nv : k);
  // fewer candidates than kk (the estimate was above the kk-th key) or more than the list holds:
  // index_rescan_kernel finishes the query
  const uint32_t nc = ws.ctr(slot)[1];
  if (kk > 0 && (nc < (uint32_t)kk || nc > ws.tie_cap)) return;
  __shared__ uint64_t keys[kSortCap];
  __shared__ uint32_t dh[256];
  __shared__ uint32_t cnt[kBins], cur[kBins];
  finalize_slot<1024>(slot, N, k, kk, idx_out, score_out, ws, keys, dh, bin_bits, cnt, cur);
}

// ---- prefill: a query the estimate did not serve ---------------------------------------------
// One workgroup per slot; every slot whose candidate list holds between kk keys and the list's
// capacity returns at once (index_sort_kernel finished it). For the others the workgroup finds
// the kk-th largest key T by a radix select over fresh passes across the query's visible keys,
// 11 key bits a pass, and a last pass collects the keys >= T: exactly the top-kk, sorted in LDS.
// The scores come from the same MFMA tiles as the select pass (every column of the B operand holds
// this query, and lanes 0..3 of each 16-lane group take keys 4 * group + 0..3), so they are the
// same values.
constexpr int kRescanDigit = 11;
constexpr int kRescanThreads = 256;

template <int HP, typename F>
__device__ __forceinline__ void rescan_keys(const QueryOps<HP>& qo,
                                            const uint8_t* __restrict__ k_codes,
                                            const uint8_t* __restrict__ k_scales,
                                            const EntryMap& kmap, int b, int64_t nv, F visit) {
  constexpr int U = 4, NW = kRescanThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, blk = lane >> 4;
  const int64_t ntile = (nv + 15) / 16;
  for (int64_t t0 = wave; t0 < ntile; t0 += NW * U) {
    u32x4 c[U];
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      int64_t g = 16 * (t0 + NW * u) + n;
      g = g < nv ? g : nv - 1;  // rows past the visible keys read a valid row (masked below)
      const int64_t row = kmap.row(b, g);
      c[u] = *(const u32x4*)(k_codes + row * 64 + 16 * blk);
      e[u] = k_scales[row * 4 + blk];
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t tile = t0 + NW * u;
      f32x4 sc = tile_scores<HP>(c[u], e[u], qo);
#pragma unroll
      for (int j = 0; j < 4; j++) sc[j] += 0.0f;  // fold -0 into +0
      const float s = n == 0 ? sc[0] : (n == 1 ? sc[1] : (n == 2 ? sc[2] : sc[3]));
      const int64_t g = 16 * tile + 4 * blk + n;
      if (n < 4 && g < nv)
        visit(((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)g));
    }
  }
}

template <int HP, bool PAGED>
__global__ __launch_bounds__(kRescanThreads) void index_rescan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, int HI,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, EntryMap kmap,
    int64_t N, const int64_t* __restrict__ pos, int m, int Q, int k,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out, IdxWs ws) {
  const int slot = blockIdx.x, b = slot / Q, i = slot - b * Q, t = threadIdx.x;
  const int64_t nv = visible_entries(pos, b, i, m, N);
  const int kk = (int)(nv < k ? nv : k);
  const uint32_t* ctr = ws.ctr(slot);
  const uint32_t nc = ctr[1];
  if (kk == 0 || (nc >= (uint32_t)kk && nc <= ws.tie_cap)) return;  // uniform over the workgroup
  constexpr int kDBins = 1 << kRescanDigit;
  constexpr int kPer = kDBins / kRescanThreads;  // digit bins per thread
  __shared__ uint32_t hist[kDBins];
  __shared__ uint32_t suf[kRescanThreads];
  __shared__ uint64_t keys[kSortCap];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ uint32_t s_r, s_cnt;
  QueryOps<HP> qo;
  load_query_ops<HP>(q_codes, q_scales, HI, (int64_t)b * Q + i, true, (t & 63) >> 4, qo);
  if (t == 0) {
    s_prefix = 0;
    s_mask = 0;
    s_r = (uint32_t)kk;  // rank (from 1) of T among all the visible keys
  }
  __syncthreads();
  for (int lo = 64; lo > 0;) {
    const int width = lo >= kRescanDigit ? kRescanDigit : lo;
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int j = t; j < kDBins; j += kRescanThreads) hist[j] = 0u;
    __syncthreads();
    // read before the barriers below; one thread rewrites them after the last of those
    const uint64_t pm = s_mask, pv = s_prefix;
    const uint32_t r = s_r;
    rescan_keys<HP>(qo, k_codes, k_scales, kmap, b, nv, [&](uint64_t x) {
      if ((x & pm) == pv) atomicAdd(&hist[(uint32_t)(x >> shift) & dmask], 1u);
    });
    __syncthreads();
    // thread t owns digits [kPer t, kPer t + kPer); suf[t] = keys in digits >= kPer t
    uint32_t own = 0;
#pragma unroll
    for (int j = 0; j < kPer; j++) own += hist[kPer * t + j];
    suf[t] = own;
    __syncthreads();
    for (int off = 1; off < kRescanThreads; off <<= 1) {
      const uint32_t v = suf[t] + (t + off < kRescanThreads ? suf[t + off] : 0u);
      __syncthreads();
      suf[t] = v;
      __syncthreads();
    }
    const uint32_t above = t + 1 < kRescanThreads ? suf[t + 1] : 0u;
    if (above < r && r <= suf[t]) {  // exactly one thread: the r-th largest is in its digits
      uint32_t cum = above;
      int d = kPer * t + kPer - 1;
      for (; d > kPer * t; d--) {
        if (cum + hist[d] >= r) break;
        cum += hist[d];
      }
      s_r = r - cum;
      s_prefix = pv | ((uint64_t)d << shift);
      s_mask = pm | ((uint64_t)dmask << shift);
    }
    __syncthreads();
    lo = shift;
  }
  // s_prefix is now T itself (all 64 bits fixed); the keys >= T are the top kk
  const uint64_t T = s_prefix;
  if (t == 0) s_cnt = 0u;
  __syncthreads();
  rescan_keys<HP>(qo, k_codes, k_scales, kmap, b, nv, [&](uint64_t x) {
    if (x >= T) {
      const uint32_t at = atomicAdd(&s_cnt, 1u);
      if (at < (uint32_t)kSortCap) keys[at] = x;
    }
  });
  __syncthreads();
  const int n = (int)(s_cnt < (uint32_t)kSortCap ? s_cnt : (uint32_t)kSortCap);
  int p2 = 2;
  while (p2 < n) p2 <<= 1;
  for (int j = n + t; j < p2; j += kRescanThreads) keys[j] = 0;
  __syncthreads();
  bitonic_sort_desc(keys, p2);
  int32_t* io = idx_out + (int64_t)slot * k;
  float* so = score_out ? score_out + (int64_t)slot * k : nullptr;
  for (int j = t; j < k; j += kRescanThreads) {
    if (j < kk && j < n) {
      const uint64_t x = keys[j];
      io[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)x);
      if (so) so[j] = key_to_float((uint32_t)(x >> 32));
    } else {
      io[j] = -1;
      if (so) so[j] = -INFINITY;
    }
  }
}

// Key ranges of at most kPKeys keys (for paged keys also at most 1024 pages, +2 partial ones, so
// that the page list fits); while the grid would be small (few sequences x query blocks), more
// and shorter ranges, down to 1024 keys, bring it to about CSAH_MFMA_WGS workgroups.
#ifndef CSAH_MFMA_WGS
#define CSAH_MFMA_WGS 512
#endif
static MfmaSplit mfma_split(const IndexArgs& a, bool paged) {
  const int64_t range_cap =
      paged ? (kPKeys < ((int64_t)1024 << a.kmap.shift) ? kPKeys : ((int64_t)1024 << a.kmap.shift))
            : kPKeys;
  MfmaSplit sp;
  sp.nqb = (a.Q + 15) / 16;
  sp.B = a.B;
  sp.nkr = 8 * (int)((a.N + 8 * range_cap - 1) / (8 * range_cap));
  if (sp.nkr < 8) sp.nkr = 8;
  int64_t want = 8 * ((CSAH_MFMA_WGS + 8LL * sp.nqb * a.B - 1) / (8LL * sp.nqb * a.B));
  const int64_t most = 8 * ((a.N + 8 * 1024 - 1) / (8 * 1024));
  if (want > most) want = most;
  if (want > sp.nkr) sp.nkr = (int)want;
  sp.keys_per_range = ((a.N + sp.nkr - 1) / sp.nkr + 15) / 16 * 16;
  return sp;
}

template <int HP, bool PAGED>
static hipError_t launch_mfma_hp(const IndexArgs& a, const IdxWs& w, hipStream_t s) {
  const int slots = a.B * a.Q;
  const MfmaSplit sp = mfma_split(a, PAGED);
  const dim3 grid((unsigned)((int64_t)sp.nkr * sp.nqb * a.B));
  index_clear_kernel<<<slots, 256, 0, s>>>(w);
  index_mfma_sample_kernel<HP, PAGED><<<(unsigned)(kSampleGroups * sp.nqb * a.B), 256, 0, s>>>(
      a.q_codes, a.q_scales, a.HI, a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, sp.nqb, w);
  index_sample_thresh_kernel<<<(slots + 3) / 4, 256, 0, s>>>(a.pos, a.m, a.Q, a.N, a.k, slots, w);
  a.prof.launch(index_mfma_select_kernel<HP, PAGED>, grid, dim3(256), s, a.q_codes, a.q_scales,
                a.HI, a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, sp, w);
  index_sort_kernel<<<slots, 1024, 0, s>>>(a.pos, a.m, a.Q, a.N, a.k, a.idx_out, a.score_out, w, 0);
  if (a.N > kSortCap)  // otherwise every query takes all its keys and no list can fall short
    index_rescan_kernel<HP, PAGED><<<slots, kRescanThreads, 0, s>>>(
        a.q_codes, a.q_scales, a.HI, a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, a.k,
        a.idx_out, a.score_out, w);
  return hipGetLastError();
}

static hipError_t launch_index_mfma(const IndexArgs& a) {
  hipStream_t s = (hipStream_t)a.stream;
  const IdxWs w = make_ws(a.ws, a.N, a.k, false);
  if (a.kmap.table) {
    if (a.HI <= 4) return launch_mfma_hp<4, true>(a, w, s);
    if (a.HI <= 8) return launch_mfma_hp<8, true>(a, w, s);
    return launch_mfma_hp<16, true>(a, w, s);
  }
  if (a.HI <= 4) return launch_mfma_hp<4, false>(a, w, s);
  if (a.HI <= 8) return launch_mfma_hp<8, false>(a, w, s);
  return launch_mfma_hp<16, false>(a, w, s);
}

template <int HP, bool PAGED>
static void launch_mfma_scan_hp(const IndexArgs& a, const IdxWs& w, hipStream_t s) {
  const MfmaSplit sp = mfma_split(a, PAGED);
  const dim3 grid((unsigned)((int64_t)sp.nkr * sp.nqb * a.B));
  a.prof.launch(index_mfma_scan_kernel<HP, PAGED>, grid, dim3(256), s, a.q_codes, a.q_scales,
                a.HI, a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, sp, w);
}

static void launch_mfma_scan(const IndexArgs& a, const IdxWs& w, hipStream_t s) {
  if (a.kmap.table) {
    if (a.HI <= 4) launch_mfma_scan_hp<4, true>(a, w, s);
    else if (a.HI <= 8) launch_mfma_scan_hp<8, true>(a, w, s);
    else launch_mfma_scan_hp<16, true>(a, w, s);
  } else {
    if (a.HI <= 4) launch_mfma_scan_hp<4, false>(a, w, s);
    else if (a.HI <= 8) launch_mfma_scan_hp<8, false>(a, w, s);
    else launch_mfma_scan_hp<16, false>(a, w, s);
  }
}

template <int NB>
static void launch_scan(const IndexArgs& a, const IdxWs& w, int chunk, dim3 grid, hipStream_t s) {
  if (NB == 4 && a.HI <= 4) {  // 128-dim keys, at most 4 heads: the MFMA scan
    if (a.kmap.table)
      a.prof.launch(index_scan_mx_kernel<true>, grid, dim3(256), s, a.q_codes, a.q_scales, a.HI,
                    a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, chunk, w);
    else
      a.prof.launch(index_scan_mx_kernel<false>, grid, dim3(256), s, a.q_codes, a.q_scales, a.HI,
                    a.k_codes, a.k_scales, a.kmap, a.N, a.pos, a.m, a.Q, chunk, w);
    return;
  }
  if (a.kmap.table)
    a.prof.launch(index_scan_kernel<NB, true>, grid, dim3(256), s, a.k_codes, a.k_scales, a.kmap,
                  a.N, a.pos, a.m, a.Q, chunk, w);
  else
    a.prof.launch(index_scan_kernel<NB, false>, grid, dim3(256), s, a.k_codes, a.k_scales, a.kmap,
                  a.N, a.pos, a.m, a.Q, chunk, w);
}

hipError_t launch_index_topk(const IndexArgs& a) {
  hipStream_t s = (hipStream_t)a.stream;
  const int slots = a.B * a.Q;
  if (use_mfma_path(a.Q, a.HI, a.dI)) return launch_index_mfma(a);
  if (use_cand(a.Q, a.HI, a.dI)) {
    CandPlan p;
    if (index_cand_plan(slots, a.N, a.k, a.kmap.table ? a.kmap.shift : -1, &p))
      return launch_index_cand(a, p);
  }
  if (use_mfma_scan(a.Q, a.HI, a.dI) && a.Q <= kCandMqMaxQ) {
    CandPlan p;
    if (index_cand_plan_mq(a.B, a.Q, a.N, a.k, a.kmap.table ? a.kmap.shift : -1, &p))
      return launch_index_cand_mq(a, p);
  }
  IdxWs w = make_ws(a.ws, a.N, a.k, true);
  index_prep_kernel<<<slots, 256, 0, s>>>(a.q_codes, a.q_scales, a.HI, a.dI, w);
  const bool mq = use_mfma_scan(a.Q, a.HI, a.dI);
  if (mq) {
    launch_mfma_scan(a, w, s);
  } else {
  // scan: about CSAH_SCAN_WGS workgroups in total, each streaming a contiguous range
  const int64_t total = (int64_t)slots * (a.N > 0 ? a.N : 1);
  int64_t chunk = (total + CSAH_SCAN_WGS - 1) / CSAH_SCAN_WGS;
  chunk = ((chunk + 1023) / 1024) * 1024;
  if (chunk < 1024) chunk = 1024;
  if (chunk > (1 << 22)) chunk = 1 << 22;
  // paged keys: a chunk spans at most 1024 pages (+1 partial one), which fits the page list
  if (a.kmap.table && chunk > ((int64_t)1024 << a.kmap.shift)) chunk = (int64_t)1024 << a.kmap.shift;
  const int64_t nchunks = a.N > 0 ? (a.N + chunk - 1) / chunk : 1;
  dim3 gs((unsigned)nchunks, (unsigned)slots);
  switch (a.dI) {
    case 32: launch_scan<1>(a, w, (int)chunk, gs, s); break;
    case 64: launch_scan<2>(a, w, (int)chunk, gs, s); break;
    default: launch_scan<4>(a, w, (int)chunk, gs, s); break;
  }
  }
  const int64_t nsel = a.N > 0 ? (a.N + kSelChunk - 1) / kSelChunk : 1;
  const dim3 gsel((unsigned)nsel, (unsigned)slots);
  if (mq)
    index_select_kernel<kPBins, kPBinShift><<<gsel, kSelThreads, 0, s>>>(a.pos, a.m, a.Q, a.N,
                                                                        a.k, w);
  else
    index_select_kernel<kBins, kBinShift><<<gsel, kSelThreads, 0, s>>>(a.pos, a.m, a.Q, a.N, a.k,
                                                                      w);
  const int64_t cand = (a.N < kSortCap ? a.N : kSortCap);
  const int64_t nrank = (cand + kRankPerWG - 1) / kRankPerWG;
  index_rank_kernel<<<dim3(nrank > 0 ? (unsigned)nrank : 1u, (unsigned)slots), kRankThreads, 0, s>>>(
      a.pos, a.m, a.Q, a.N, a.k, a.idx_out, a.score_out, w, 32 - (mq ? kPBinShift : kBinShift));
  return hipGetLastError();
}

}  // namespace csah
