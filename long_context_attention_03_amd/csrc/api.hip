// api.hip -- the C ABI declared in include/csah.h: argument validation, workspace sizing, device
// check and kernel launches. Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "csah_internal.h"

using namespace csah;

namespace {

// Validation never touches the HIP runtime; the device check runs only for valid arguments.
int check_device() {
  static std::mutex mu;
  static int cached[64];
  static bool init[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return CSAH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (!init[dev]) {
    hipDeviceProp_t prop;
    int ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
             strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cached[dev] = ok ? CSAH_OK : CSAH_ERR_UNSUPPORTED;
    init[dev] = true;
  }
  return cached[dev];
}

int launch_status(hipError_t e) { return e == hipSuccess ? CSAH_OK : CSAH_ERR_LAUNCH; }

// Scratch of csah_csa_attend_noalloc: the split partials live in this array instead of a caller
// workspace. Every GPU the library runs on holds its own copy until the process ends. In host
// code the name is only a stand-in: kernels get the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device on its first call.
static __device__ __align__(256) unsigned char scratch[CSAH_NOALLOC_SCRATCH_BYTES];

void* scratch_address() {
  static std::mutex mu;
  static void* addr[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!done[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    addr[dev] = ptr;
    done[dev] = true;
  }
  return addr[dev];
}

thread_local ProfileHook g_next_prof;

// Take (and clear) this thread's pending profiling request.
ProfileHook take_profile() {
  ProfileHook h = g_next_prof;
  g_next_prof = ProfileHook{};
  return h;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A block-table layout: page_size is a power of two in [1, 2^20]; `capacity` receives the
// entries each sequence's table row can address (table_stride pages).
int paged_map(const int32_t* table, int64_t table_stride, int page_size, EntryMap& map,
              int64_t& capacity) {
  if (!table || !aligned(table, 4) || page_size <= 0 || (page_size & (page_size - 1)) != 0 ||
      table_stride < 0)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (page_size > (1 << 20)) return CSAH_ERR_UNSUPPORTED;
  int shift = 0;
  while ((1 << shift) < page_size) shift++;
  if (table_stride > (INT64_MAX >> 21)) return CSAH_ERR_INVALID_ARGUMENT;
  map = EntryMap{table, table_stride, shift};
  capacity = table_stride << shift;
  return CSAH_OK;
}

EntryMap contiguous_map(int64_t seq_stride) { return EntryMap{nullptr, seq_stride, 0}; }

// RoPE widths: an even number of rotary dims 2 <= R <= D, D even (pairs stay aligned), and a
// finite positive base.
bool rope_shape_ok(int D, int R, double base) {
  return D % 2 == 0 && R >= 2 && R % 2 == 0 && R <= D && base > 0.0 && base < INFINITY;
}

int row_bytes(int fmt, int D) {
  if (fmt == CSAH_FMT_ROW_F32) return 4 * D;
  if (fmt == CSAH_FMT_ROW_E4M3_BF16) return D >= 64 ? D + 64 : -1;
  if (fmt == CSAH_FMT_FP4_E8M0) return D % 2 == 0 ? D / 2 : -1;
  return -1;
}

}  // namespace

extern "C" {

int csah_abi_version(void) { return CSAH_ABI_VERSION; }

const char* csah_status_string(int status) {
  switch (status) {
    case CSAH_OK: return "ok";
    case CSAH_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CSAH_ERR_UNSUPPORTED: return "unsupported shape, format or device";
    case CSAH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CSAH_ERR_LAUNCH: return "kernel launch failed";
    case CSAH_ERR_SCRATCH_LIMIT:
      return "the call needs more than the library's static scratch (CSAH_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int64_t csah_row_bytes(int fmt, int D) { return D > 0 ? row_bytes(fmt, D) : -1; }

int csah_profile_next_call(void* begin_event, void* end_event) {
  if ((begin_event == nullptr) != (end_event == nullptr)) return CSAH_ERR_INVALID_ARGUMENT;
  g_next_prof.begin = (hipEvent_t)begin_event;
  g_next_prof.end = (hipEvent_t)end_event;
  return CSAH_OK;
}

// out_capacity: output entries each sequence can take from first_entry on.
static int kv_compress_impl(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                            int64_t T, int D, int m, int span, int64_t skip, const float* w,
                            const float* beta, void* out_rows, int out_fmt, EntryMap out_map,
                            int64_t first_entry, int64_t out_capacity, uint8_t* out_scales,
                            void* stream, ProfileHook prof, const int64_t* tok_pos = nullptr,
                            int rope_dims = 0, double rope_base = 0.0) {
  if (B < 0 || T < 0 || D <= 0 || m <= 0) return CSAH_ERR_INVALID_ARGUMENT;
  if (rope_dims != 0 && !rope_shape_ok(D, rope_dims, rope_base)) return CSAH_ERR_INVALID_ARGUMENT;
  if (raw_dtype != CSAH_DT_F32 && raw_dtype != CSAH_DT_BF16) return CSAH_ERR_INVALID_ARGUMENT;
  if (out_fmt != CSAH_FMT_ROW_F32 && out_fmt != CSAH_FMT_ROW_E4M3_BF16 &&
      out_fmt != CSAH_FMT_FP4_E8M0)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (T % m != 0 || span < m || skip < 0 || skip > T / m || raw_seq_stride < T ||
      out_capacity < T / m - skip)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (B == 0 || T / m - skip == 0) return CSAH_OK;  // no entry to write: nothing is touched
  if (!raw || !w || !beta || !out_rows) return CSAH_ERR_INVALID_ARGUMENT;
  if ((out_fmt == CSAH_FMT_FP4_E8M0) != (out_scales != nullptr)) return CSAH_ERR_INVALID_ARGUMENT;
  if (!aligned(raw, 16) || !aligned(out_rows, 16)) return CSAH_ERR_INVALID_ARGUMENT;
  if (D != 64 && D != 128 && D != 256 && D != 512 && D != 1024) return CSAH_ERR_UNSUPPORTED;
  if (out_fmt == CSAH_FMT_ROW_E4M3_BF16 && D != 512) return CSAH_ERR_UNSUPPORTED;
  if (span > 65536) return CSAH_ERR_UNSUPPORTED;
  if (rope_dims != 0 && (!tok_pos || !aligned(tok_pos, 8))) return CSAH_ERR_INVALID_ARGUMENT;
  int st = check_device();
  if (st) return st;
  KvCompressArgs a{raw,  raw_dtype, raw_seq_stride, B,       T / m - skip, D,          m,
                   span, skip,      w,              beta,    out_rows,     out_fmt,    out_map,
                   first_entry,     out_scales,     stream,  prof};
  a.tok_pos = tok_pos;
  a.rope_dims = rope_dims;
  a.rope_base = rope_base;
  return launch_status(launch_kv_compress(a));
}

int csah_kv_compress(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B, int64_t T,
                     int D, int m, const float* w, const float* beta, void* out_rows, int out_fmt,
                     int64_t out_seq_stride, uint8_t* out_scales, void* stream) {
  const ProfileHook prof = take_profile();
  return kv_compress_impl(raw, raw_dtype, raw_seq_stride, B, T, D, m, m, 0, w, beta, out_rows,
                          out_fmt, contiguous_map(out_seq_stride), 0, out_seq_stride, out_scales,
                          stream, prof);
}

int csah_kv_compress_span(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                          int64_t T, int D, int m, int span, int64_t skip, const float* w,
                          const float* beta, void* out_rows, int out_fmt, int64_t out_seq_stride,
                          uint8_t* out_scales, void* stream) {
  const ProfileHook prof = take_profile();
  return kv_compress_impl(raw, raw_dtype, raw_seq_stride, B, T, D, m, span, skip, w, beta,
                          out_rows, out_fmt, contiguous_map(out_seq_stride), 0, out_seq_stride,
                          out_scales, stream, prof);
}

int csah_kv_compress_paged(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                           int64_t T, int D, int m, int span, int64_t skip, const float* w,
                           const float* beta, void* out_pool, int out_fmt,
                           uint8_t* out_scale_pool, const int32_t* block_table,
                           int64_t table_stride, int page_size, int64_t first_entry,
                           void* stream) {
  const ProfileHook prof = take_profile();
  EntryMap map;
  int64_t cap;
  const int st = paged_map(block_table, table_stride, page_size, map, cap);
  if (st) return st;
  if (first_entry < 0 || first_entry > cap) return CSAH_ERR_INVALID_ARGUMENT;
  return kv_compress_impl(raw, raw_dtype, raw_seq_stride, B, T, D, m, span, skip, w, beta,
                          out_pool, out_fmt, map, first_entry, cap - first_entry, out_scale_pool,
                          stream, prof);
}

int csah_kv_compress_rope(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                          int64_t T, int D, int m, int span, int64_t skip, const float* w,
                          const float* beta, void* out_rows, int out_fmt, int64_t out_seq_stride,
                          uint8_t* out_scales, const int64_t* tok_pos, int rope_dims,
                          double rope_base, void* stream) {
  const ProfileHook prof = take_profile();
  if (rope_dims == 0) return CSAH_ERR_INVALID_ARGUMENT;
  return kv_compress_impl(raw, raw_dtype, raw_seq_stride, B, T, D, m, span, skip, w, beta,
                          out_rows, out_fmt, contiguous_map(out_seq_stride), 0, out_seq_stride,
                          out_scales, stream, prof, tok_pos, rope_dims, rope_base);
}

int csah_kv_compress_paged_rope(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                                int64_t T, int D, int m, int span, int64_t skip, const float* w,
                                const float* beta, void* out_pool, int out_fmt,
                                uint8_t* out_scale_pool, const int32_t* block_table,
                                int64_t table_stride, int page_size, int64_t first_entry,
                                const int64_t* tok_pos, int rope_dims, double rope_base,
                                void* stream) {
  const ProfileHook prof = take_profile();
  if (rope_dims == 0) return CSAH_ERR_INVALID_ARGUMENT;
  EntryMap map;
  int64_t cap;
  const int st = paged_map(block_table, table_stride, page_size, map, cap);
  if (st) return st;
  if (first_entry < 0 || first_entry > cap) return CSAH_ERR_INVALID_ARGUMENT;
  return kv_compress_impl(raw, raw_dtype, raw_seq_stride, B, T, D, m, span, skip, w, beta,
                          out_pool, out_fmt, map, first_entry, cap - first_entry, out_scale_pool,
                          stream, prof, tok_pos, rope_dims, rope_base);
}

int csah_rope(void* x, int dtype, int B, int Q, int H, int D, int rope_dims, const int64_t* pos,
              double rope_base, int inverse, void* stream) {
  const ProfileHook prof = take_profile();
  if (B < 0 || Q < 0 || H <= 0 || D <= 0 || (inverse != 0 && inverse != 1))
    return CSAH_ERR_INVALID_ARGUMENT;
  if (dtype != CSAH_DT_F32 && dtype != CSAH_DT_BF16) return CSAH_ERR_INVALID_ARGUMENT;
  if (!rope_shape_ok(D, rope_dims, rope_base)) return CSAH_ERR_INVALID_ARGUMENT;
  if (rope_dims > 2 * kRopeMaxPairs) return CSAH_ERR_UNSUPPORTED;
  // the kernels count a row group's pairs and vectors in 32-bit integers
  if ((int64_t)B * Q > INT32_MAX || (int64_t)H * rope_dims > (1 << 28)) return CSAH_ERR_UNSUPPORTED;
  if (B == 0 || Q == 0) return CSAH_OK;  // no row: nothing is touched
  if (!x || !pos || !aligned(x, 16) || !aligned(pos, 8)) return CSAH_ERR_INVALID_ARGUMENT;
  int st = check_device();
  if (st) return st;
  RopeArgs a{x, dtype, B, Q, H, D, rope_dims, pos, rope_base, inverse, stream, prof};
  return launch_status(launch_rope(a));
}

size_t csah_index_topk_workspace(int B, int Q, int64_t N, int k, int HI, int dI) {
  if (B <= 0 || Q <= 0 || N < 0 || k <= 0 || HI <= 0) return 0;
  return index_workspace_bytes(B, Q, N, k, HI, dI);
}

// capacity: entries each sequence's keys can hold (the row stride, or what the table covers).
static int index_impl(const uint8_t* q_codes, const uint8_t* q_scales, int HI, int dI,
                      const uint8_t* k_codes, const uint8_t* k_scales, EntryMap kmap,
                      int64_t capacity, int64_t N, const int64_t* pos, int m, int B, int Q, int k,
                      int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes, void* stream,
                      ProfileHook prof) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !pos || !idx_out || !ws)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (HI <= 0 || dI <= 0 || m <= 0 || B <= 0 || Q <= 0 || k <= 0 || N < 0 || capacity < N)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(ws, 256))
    return CSAH_ERR_INVALID_ARGUMENT;
  if (HI > 16 || (dI != 32 && dI != 64 && dI != 128) || k > 4096 || N >= ((int64_t)1 << 31) ||
      (int64_t)B * Q >= 65536)
    return CSAH_ERR_UNSUPPORTED;
  int st = check_device();
  if (st) return st;
  if (ws_bytes < index_workspace_bytes(B, Q, N, k, HI, dI)) return CSAH_ERR_WORKSPACE_TOO_SMALL;
  IndexArgs a{q_codes, q_scales, HI, dI, k_codes, k_scales, kmap, N, pos, m, B, Q, k,
              idx_out, score_out, ws, ws_bytes, stream, prof};
  return launch_status(launch_index_topk(a));
}

int csah_index_topk(const uint8_t* q_codes, const uint8_t* q_scales, int HI, int dI,
                    const uint8_t* k_codes, const uint8_t* k_scales, int64_t k_seq_stride,
                    int64_t N, const int64_t* pos, int m, int B, int Q, int k, int32_t* idx_out,
                    float* score_out, void* ws, size_t ws_bytes, void* stream) {
  const ProfileHook prof = take_profile();
  return index_impl(q_codes, q_scales, HI, dI, k_codes, k_scales, contiguous_map(k_seq_stride),
                    k_seq_stride, N, pos, m, B, Q, k, idx_out, score_out, ws, ws_bytes, stream,
                    prof);
}

int csah_index_topk_paged(const uint8_t* q_codes, const uint8_t* q_scales, int HI, int dI,
                          const uint8_t* k_pool_codes, const uint8_t* k_pool_scales,
                          const int32_t* block_table, int64_t table_stride, int page_size,
                          int64_t N, const int64_t* pos, int m, int B, int Q, int k,
                          int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes,
                          void* stream) {
  const ProfileHook prof = take_profile();
  EntryMap map;
  int64_t cap;
  const int st = paged_map(block_table, table_stride, page_size, map, cap);
  if (st) return st;
  return index_impl(q_codes, q_scales, HI, dI, k_pool_codes, k_pool_scales, map, cap, N, pos, m,
                    B, Q, k, idx_out, score_out, ws, ws_bytes, stream, prof);
}

size_t csah_attend_workspace(int B, int Q, int H, int D, int64_t max_rows) {
  if (B <= 0 || Q <= 0 || H <= 0 || D <= 0 || max_rows < 0) return 0;
  return attend_workspace_bytes(B, Q, H, D, max_rows);
}

static int attend_common(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                         EntryMap cmap, int64_t capacity, int64_t N, const int32_t* idx, int k, int m,
                         const void* win, int64_t win_seq_stride, int w, const int64_t* pos,
                         const float* sink, float scale, int B, int Q, float* out, float* lse,
                         void* ws, size_t ws_bytes, void* stream, ProfileHook prof) {
  if (!q || !cache || !pos || !out || H <= 0 || D <= 0 || B <= 0 || Q <= 0 || N < 0 || w < 0)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (q_dtype != CSAH_DT_F32 && q_dtype != CSAH_DT_BF16) return CSAH_ERR_INVALID_ARGUMENT;
  if (fmt != CSAH_FMT_ROW_F32 && fmt != CSAH_FMT_ROW_E4M3_BF16) return CSAH_ERR_INVALID_ARGUMENT;
  if (capacity < N) return CSAH_ERR_INVALID_ARGUMENT;
  if (w > 0 && (!win || win_seq_stride < (int64_t)w - 1 + Q)) return CSAH_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(cache, 16) || (w > 0 && !aligned(win, 16)))
    return CSAH_ERR_INVALID_ARGUMENT;
  if (!((fmt == CSAH_FMT_ROW_E4M3_BF16 && D == 512) || (fmt == CSAH_FMT_ROW_F32 && D == 128)))
    return CSAH_ERR_UNSUPPORTED;
  const int64_t max_rows = (idx ? (int64_t)k : N) + w;
  if (max_rows >= ((int64_t)1 << 31) || (int64_t)B * Q >= 65536) return CSAH_ERR_UNSUPPORTED;
  int st = check_device();
  if (st) return st;
  const size_t need = attend_workspace_bytes(B, Q, H, D, max_rows);
  if (need > 0 && (!ws || !aligned(ws, 256))) return need > ws_bytes ? CSAH_ERR_WORKSPACE_TOO_SMALL
                                                                       : CSAH_ERR_INVALID_ARGUMENT;
  if (ws_bytes < need) return CSAH_ERR_WORKSPACE_TOO_SMALL;
  AttendArgs a{q,   q_dtype, H,     D,     cache, fmt, cmap,             N,        idx,   k,
               m,   win,     win_seq_stride, w, pos, sink, scale,   B,  Q, out, lse, ws, ws_bytes,
               stream, max_rows, prof};
  return launch_status(launch_attend(a));
}

int csah_csa_attend(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                    int64_t cache_seq_stride, int64_t N, const int32_t* idx, int k,
                    const void* win, int64_t win_seq_stride, int w, const int64_t* pos,
                    const float* sink, float scale, int B, int Q, float* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
  const ProfileHook prof = take_profile();
  if (!idx || k < 0) return CSAH_ERR_INVALID_ARGUMENT;
  return attend_common(q, q_dtype, H, D, cache, fmt, contiguous_map(cache_seq_stride),
                       cache_seq_stride, N, idx, k, 1, win,
                       win_seq_stride, w, pos, sink, scale, B, Q, out, lse, ws, ws_bytes, stream,
                       prof);
}

int csah_csa_attend_noalloc(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                            int64_t cache_seq_stride, int64_t N, const int32_t* idx, int k,
                            const void* win, int64_t win_seq_stride, int w, const int64_t* pos,
                            const float* sink, float scale, int B, int Q, float* out, float* lse,
                            void* stream) {
  const ProfileHook prof = take_profile();
  if (!idx || k < 0 || w < 0 || H <= 0 || D <= 0 || B <= 0 || Q <= 0)
    return CSAH_ERR_INVALID_ARGUMENT;
  if (attend_workspace_bytes(B, Q, H, D, (int64_t)k + w) > CSAH_NOALLOC_SCRATCH_BYTES)
    return CSAH_ERR_SCRATCH_LIMIT;
  int st = check_device();
  if (st) return st;
  void* ws = scratch_address();
  if (!ws) return CSAH_ERR_LAUNCH;
  return attend_common(q, q_dtype, H, D, cache, fmt, contiguous_map(cache_seq_stride),
                       cache_seq_stride, N, idx, k, 1, win, win_seq_stride, w, pos, sink, scale,
                       B, Q, out, lse, ws, CSAH_NOALLOC_SCRATCH_BYTES, stream, prof);
}

int csah_hca_attend(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                    int64_t cache_seq_stride, int64_t N, int m, const void* win,
                    int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                    float scale, int B, int Q, float* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  const ProfileHook prof = take_profile();
  if (m <= 0) return CSAH_ERR_INVALID_ARGUMENT;
  return attend_common(q, q_dtype, H, D, cache, fmt, contiguous_map(cache_seq_stride),
                       cache_seq_stride, N, nullptr, 0, m, win,
                       win_seq_stride, w, pos, sink, scale, B, Q, out, lse, ws, ws_bytes, stream,
                       prof);
}

int csah_csa_attend_paged(const void* q, int q_dtype, int H, int D, const void* cache_pool,
                          int fmt, const int32_t* block_table, int64_t table_stride,
                          int page_size, int64_t N, const int32_t* idx, int k, const void* win,
                          int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                          float scale, int B, int Q, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream) {
  const ProfileHook prof = take_profile();
  if (!idx || k < 0) return CSAH_ERR_INVALID_ARGUMENT;
  EntryMap map;
  int64_t cap;
  const int st = paged_map(block_table, table_stride, page_size, map, cap);
  if (st) return st;
  return attend_common(q, q_dtype, H, D, cache_pool, fmt, map, cap, N, idx, k, 1, win,
                       win_seq_stride, w, pos, sink, scale, B, Q, out, lse, ws, ws_bytes, stream,
                       prof);
}

int csah_hca_attend_paged(const void* q, int q_dtype, int H, int D, const void* cache_pool,
                          int fmt, const int32_t* block_table, int64_t table_stride,
                          int page_size, int64_t N, int m, const void* win,
                          int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                          float scale, int B, int Q, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream) {
  const ProfileHook prof = take_profile();
  if (m <= 0) return CSAH_ERR_INVALID_ARGUMENT;
  EntryMap map;
  int64_t cap;
  const int st = paged_map(block_table, table_stride, page_size, map, cap);
  if (st) return st;
  return attend_common(q, q_dtype, H, D, cache_pool, fmt, map, cap, N, nullptr, 0, m, win,
                       win_seq_stride, w, pos, sink, scale, B, Q, out, lse, ws, ws_bytes, stream,
                       prof);
}

}  // extern "C"
