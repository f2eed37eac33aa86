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

}  // namespace csah
