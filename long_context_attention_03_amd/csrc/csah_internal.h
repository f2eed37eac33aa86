// csah_internal.h -- launch descriptors shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csah.h"

namespace csah {

// Where entry e of sequence b of a cache lives, as a row number of the array the kernel gets.
// Contiguous (table == NULL): row b * stride + e. Paged: row table[b * stride + (e >> shift)] *
// 2^shift + (e mod 2^shift), i.e. sequence b's block-table row names the pool page that holds
// its entries [2^shift * i, 2^shift * (i + 1)).
struct EntryMap {
  const int32_t* table;
  int64_t stride;  // contiguous: rows per sequence; paged: table entries per sequence
  int shift;       // paged: log2 of the page size in entries
  __device__ __forceinline__ int64_t flat(int b, int64_t e) const { return (int64_t)b * stride + e; }
  __device__ __forceinline__ int64_t paged(int b, int64_t e) const {
    const int64_t page = table[(int64_t)b * stride + (e >> shift)];
    return (page << shift) | (e & (((int64_t)1 << shift) - 1));
  }
  __device__ __forceinline__ int64_t row(int b, int64_t e) const {
    return table ? paged(b, e) : flat(b, e);
  }
};

// Events attached to the dispatch of a call's dominant kernel (both null: plain launch). The
// runtime stamps them with that dispatch's own start and end, so they time the kernel alone.
struct ProfileHook {
  hipEvent_t begin = nullptr, end = nullptr;
  template <typename... KArgs, typename... Args>
  void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
              Args... args) const {
    if (begin || end)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, s, begin, end, 0, (KArgs)args...);
    else
      kernel<<<grid, block, 0, s>>>((KArgs)args...);
  }
};

struct KvCompressArgs {
  const void* raw;
  int raw_dtype;
  int64_t raw_seq_stride;
  int B;
  int64_t G;     // entries written per sequence = T / m - skip
  int D, m;
  int span;      // tokens per entry (m: one entry per group)
  int64_t skip;  // leading groups that are context only
  const float* w;
  const float* beta;
  void* out_rows;
  int out_fmt;
  EntryMap out_map;     // where output entry first_entry + g of sequence b goes
  int64_t first_entry;  // logical index of the call's first output entry
  uint8_t* out_scales;
  void* stream;
  ProfileHook prof;
  // RoPE of the pooled entry before encoding (rope_dims = 0: none): the last rope_dims dims turn
  // at the position of the group's last token, tok_pos[b] + m (group + 1) - 1
  const int64_t* tok_pos = nullptr;
  int rope_dims = 0;
  double rope_base = 0.0;
};
hipError_t launch_kv_compress(const KvCompressArgs& a);

// ---- rope --------------------------------------------------------------------------------------
constexpr int kRopeMaxPairs = 512;  // rotary dims per row: at most 1024
struct RopeArgs {
  void* x;  // [B][Q][H][D] of dtype, turned in place
  int dtype;
  int B, Q, H, D, R;
  const int64_t* pos;  // [B]: row group (b, i) sits at pos[b] + i
  double base;
  int inverse;
  void* stream;
  ProfileHook prof;
};
hipError_t launch_rope(const RopeArgs& a);

// ---- index_topk --------------------------------------------------------------------------------
struct IndexArgs {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  int HI, dI;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  EntryMap kmap;
  int64_t N;
  const int64_t* pos;
  int m, B, Q, k;
  int32_t* idx_out;
  float* score_out;
  void* ws;
  size_t ws_bytes;
  void* stream;
  ProfileHook prof;
};
size_t index_workspace_bytes(int B, int Q, int64_t N, int k, int HI, int dI);
hipError_t launch_index_topk(const IndexArgs& a);

// One or two queries per sequence: certified per-range candidate lists and a top-k over their union
// (index_cand.hip). The plan fixes the range length (chunk), the ranges per slot (R), the list
// length (cap) and how many keys a range publishes at least (cmin).
struct CandPlan {
  int chunk, R, cap, cmin;
};
// false: more ranges than the top-k kernel holds (very long key ranges); page_shift < 0: contiguous
bool index_cand_plan(int slots, int64_t N, int k, int page_shift, CandPlan* p);
size_t index_cand_slot_bytes();
hipError_t launch_index_cand(const IndexArgs& a, const CandPlan& p);
// 3 to kCandMqMaxQ queries per sequence (128-dim keys): one MFMA pass per range scores all of a
// sequence's queries and publishes a list per query; the same top-k finishes each query. Measured
// at 4 x 262,144 keys: 34.5 / 42.4 / 46.6 / 50.3 us against 49.3 / 58.3 / 61.3 / 63.5 us (stored
// scores) for 3 / 5 / 6 / 7 queries; at 8 the LDS stage caps the ranges below 2048 keys and the
// scan needs a second round of workgroups (79.0 against 64.7 us).
constexpr int kCandMqMaxQ = 7;
bool index_cand_plan_mq(int B, int Q, int64_t N, int k, int page_shift, CandPlan* p);
hipError_t launch_index_cand_mq(const IndexArgs& a, const CandPlan& p);

// ---- attention ---------------------------------------------------------------------------------
struct AttendPlan {
  int splits;          // row splits per (sequence, query, head group)
  int rows_per_split;  // multiple of the 32-row tile
  int head_groups;     // ceil(H / 16)
};
AttendPlan attend_plan(int B, int Q, int H, int D, int64_t max_rows);
size_t attend_workspace_bytes(int B, int Q, int H, int D, int64_t max_rows);

struct AttendArgs {
  const void* q;
  int q_dtype, H, D;
  const void* cache;
  int fmt;
  EntryMap cmap;
  int64_t N;
  const int32_t* idx;  // NULL: dense (HCA) over g < floor((pos+i+1)/m)
  int k, m;
  const void* win;
  int64_t win_seq_stride;
  int w;
  const int64_t* pos;
  const float* sink;
  float scale;
  int B, Q;
  float* out;
  float* lse;
  void* ws;
  size_t ws_bytes;
  void* stream;
  int64_t max_rows;
  ProfileHook prof;
};
hipError_t launch_attend(const AttendArgs& a);

}  // namespace csah
