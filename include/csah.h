/*
 * csah.h -- C ABI of a compress-then-sparsify attention library for AMD Instinct MI355X (gfx950).
 *
 * The library implements the attention hot path of DeepSeek-V4's hybrid attention as described by
 *   [EXPL]  "DeepSeek V4 Architecture Explained: CSA, HCA, mHC and Muon", section
 *           "How compress-then-sparsify attention works" and the "Key numbers" table;
 *   [LLMB]  "Inside DeepSeek-V4: How Hybrid Sparse Attention Slashes 1M Context Overhead by 90%",
 *           sections "1. Compressed Sparse Attention (CSA)" and "2. Heavily Compressed
 *           Attention (HCA)";
 *   [BSWEN] "How DeepSeek V4 Handles 1M Token Context with Hybrid Attention", sections
 *           "Component 2: Multi-Level KV Compression" and "Component 3: DeepSeek Sparse
 *           Attention (DSA)".
 *
 * Conventions shared by every entry point
 *  - Every array argument is a DEVICE pointer to memory owned by the caller. The library never
 *    allocates, frees or synchronises. Between calls it keeps only a thread's pending profiling
 *    request (csah_profile_next_call, consumed by that thread's next call) and, for
 *    csah_csa_attend_noalloc, a scratch array in every GPU it runs on.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). A call only enqueues
 *    kernels on it and returns.
 *  - Arguments are validated on the host before anything is enqueued. On a nonzero status nothing
 *    was enqueued. Device buffers smaller than the shapes imply, or device-side values outside
 *    their documented ranges, are not detectable on the host: kernels clamp every index they
 *    derive from device data so that they stay inside the shapes passed, and the results are then
 *    unspecified.
 *  - Strides are counted in rows (tokens or entries) of the buffer's own row format.
 *  - Calls are reentrant; concurrent calls must use distinct workspaces (concurrent
 *    csah_csa_attend_noalloc calls on one GPU share its scratch and must be ordered).
 *
 * Row formats of one token's / one compressed entry's shared K=V vector (D values):
 *   CSAH_FMT_ROW_F32        D little-endian binary32 values (4*D bytes).
 *   CSAH_FMT_ROW_E4M3_BF16  D-64 OCP E4M3 bytes (unit scale) followed by 64 bf16 values
 *                           (D+64 bytes; 576 bytes at D=512). [EXPL] "Key numbers": rotary
 *                           dimensions are stored in BF16 and the others in FP8.
 *   CSAH_FMT_FP4_E8M0       indexer keys / queries: D/2 bytes of OCP MX E2M1 codes (element 2j in
 *                           the low nibble of byte j) in the row array, and D/32 E8M0 scale bytes
 *                           per row in a separate scale array indexed by the same rows.
 */
#ifndef CSAH_H
#define CSAH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSAH_ABI_VERSION 1

/* status codes */
#define CSAH_OK 0
#define CSAH_ERR_INVALID_ARGUMENT (-1) /* null pointer, bad shape or stride                   */
#define CSAH_ERR_UNSUPPORTED (-2)      /* shape/format combination not built, or no gfx950    */
#define CSAH_ERR_WORKSPACE_TOO_SMALL (-3)
#define CSAH_ERR_LAUNCH (-4)           /* the HIP runtime refused a launch                     */
#define CSAH_ERR_SCRATCH_LIMIT (-5)    /* csah_csa_attend_noalloc: more than its static scratch */

/* element types of raw rows and queries */
#define CSAH_DT_F32 0
#define CSAH_DT_BF16 1

/* row formats */
#define CSAH_FMT_ROW_F32 0
#define CSAH_FMT_ROW_E4M3_BF16 1
#define CSAH_FMT_FP4_E8M0 2

/* ABI version of the loaded library (CSAH_ABI_VERSION at build time). */
int csah_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* csah_status_string(int status);

/* Bytes per row of `fmt` at width D (the row array only for FP4_E8M0); -1 if not a format. */
int64_t csah_row_bytes(int fmt, int D);

/*
 * csah_kv_compress -- softmax-gated pooling of each group of m consecutive tokens' shared K=V row
 * into one compressed entry, with a learned bias per position inside the group.
 *   [EXPL]: m consecutive tokens fold into one KV entry through trainable compression weights, a
 *   softmax over the group and learnable positional biases. [LLMB] "1. CSA": factor 4;
 *   "2. HCA": factor 128. For group g (tokens gm .. gm+m-1):
 *     z_t = sum_c w[c] * x_t[c] + beta[t - g*m],   pi = softmax_t(z),   c_g = sum_t pi_t * x_t,
 *   then c_g is encoded in out_fmt (E4M3 and E2M1 round to nearest even and saturate; MX blocks
 *   use the shared exponent floor(log2 amax) - 2, and an all-zero block gets scale byte 127).
 *   m = 1 returns the rows themselves, encoded: it is also the library's quantiser.
 * raw       [B][raw_seq_stride][D] tokens, raw_dtype CSAH_DT_F32 or CSAH_DT_BF16; only the first T
 *           rows of each sequence are read.
 * T         tokens per sequence; must be a multiple of m (complete groups only).
 * w, beta   fp32 gate weights [D] and positional biases [m].
 * out_rows  [B][out_seq_stride] rows of out_fmt; entry g of sequence b is written to row
 *           b*out_seq_stride + g (point it at the cache's append position). out_seq_stride >= T/m.
 * out_scales FP4_E8M0 only: [B][out_seq_stride][D/32] scale bytes (NULL otherwise).
 * A call that writes no entry (B = 0 or T = 0) returns CSAH_OK after checking the scalar
 * arguments and touches no buffer; its pointers may then be NULL.
 * Supported: D in {64, 128, 256, 512, 1024}; D == 512 for ROW_E4M3_BF16; 1 <= m <= 65536.
 */
int csah_kv_compress(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B, int64_t T,
                     int D, int m, const float* w, const float* beta, void* out_rows, int out_fmt,
                     int64_t out_seq_stride, uint8_t* out_scales, void* stream);

/*
 * csah_kv_compress_span -- the same pooling with entries of `span` tokens at stride m.
 *   [BSWEN] "Component 2: Multi-Level KV Compression": one level compresses 8 tokens into one
 *   entry with a stride of 4 (span = 8, m = 4). Entry g pools the span tokens that end with the
 *   last token of group g, tokens [m(g+1) - span, m(g+1)) of raw:
 *     z_t = w . x_t + beta[t - (m(g+1) - span)],  pi = softmax over the entry's tokens,
 *     c_g = sum_t pi_t x_t,  encoded as in csah_kv_compress.
 *   Tokens before the start of raw are left out of the softmax (the start of a sequence). The
 *   first `skip` groups are context only: entry g >= skip is written to output row g - skip, so a
 *   caller appending entries passes the span - m tokens before the new groups and skip =
 *   (span - m) / m. span = m, skip = 0 is exactly csah_kv_compress.
 * beta      fp32 positional biases [span], indexed by the token's place in its span.
 * out_rows  [B][out_seq_stride] rows, out_seq_stride >= T/m - skip; T/m - skip entries written.
 * Other arguments, layouts and statuses as csah_kv_compress; also CSAH_ERR_INVALID_ARGUMENT if
 * span < m or skip > T/m, CSAH_ERR_UNSUPPORTED if span > 65536.
 */
int csah_kv_compress_span(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                          int64_t T, int D, int m, int span, int64_t skip, const float* w,
                          const float* beta, void* out_rows, int out_fmt, int64_t out_seq_stride,
                          uint8_t* out_scales, void* stream);

/*
 * csah_index_topk -- the lightning indexer: score every visible compressed entry against the
 * query's FP4 indexer heads and keep the top k.
 *   [EXPL]: low-rank indexer queries are scored against compressed indexer keys and each query
 *   keeps its top-k entries; [LLMB] "1. CSA": the indexer runs in FP4 and keeps the top 1,024;
 *   [BSWEN] "Component 3": score all compressed entries, then select the top k.
 *   score_g = sum_h sum_blocks 2^(Eq+Ek-254) * sum_{i in block} e2m1(q_h,i) * e2m1(k_g,i)
 *   (a plain sum over heads). Scores are dyadic and computed exactly whenever the sum of the
 *   absolute products over the finest power-of-two granularity stays below 2^24 and all scales
 *   keep the products inside the binary32 normal range.
 *   Query i of sequence b sees entries g < min(floor((pos[b]+i+1)/m), N): a group is visible once
 *   it is complete. The output lists the first min(k, visible) entries ordered by (score
 *   descending, index ascending); remaining slots are -1 (score -inf).
 * q_codes   [B][Q][HI][dI/2] E2M1 codes (16-byte aligned), q_scales [B][Q][HI][dI/32] E8M0.
 * k_codes   [B][k_seq_stride][dI/2], k_scales [B][k_seq_stride][dI/32]; N <= k_seq_stride.
 * pos       [B] int64 device array, position of query 0 of each sequence.
 * idx_out   [B][Q][k] int32; score_out [B][Q][k] fp32 or NULL.
 * ws        device workspace of at least csah_index_topk_workspace(B, Q, N, k, HI, dI) bytes,
 *           256-byte aligned; its contents need no initialisation and are clobbered.
 * Supported: 1 <= HI <= 16, dI in {32, 64, 128}, 1 <= k <= 4096, N < 2^31, m >= 1, B*Q < 65536.
 * Several schedules compute the same result; the workspace size follows the one the shape takes.
 *  - Decode (Q <= 2 queries per sequence, N <= 2^20): a scan leaves per-range candidate lists and
 *    one top-k pass per query ranks their union; the workspace is a fixed 73,728 bytes per
 *    (sequence, query) slot, whatever N.
 *  - dI = 128 and Q >= 16 (a prefill chunk: many queries of one sequence share its keys): the
 *    scores come from the scaled FP4 MFMA and are recomputed rather than stored; the workspace
 *    holds, per query, a histogram, counters and a candidate list of max(8192, 4k) 8-byte keys
 *    (at most N), whatever N is.
 *  - dI = 128 and 3 <= Q <= 7: one pass per key range scores all of a sequence's queries and
 *    leaves a candidate list per query, ranked as in the decode schedule; the workspace is the
 *    larger of that schedule's 73,728 bytes per slot and the stored-score one below (which
 *    serves the call when the keys span more ranges than the lists allow).
 *  - Otherwise (8 <= Q <= 15 with 128-dim keys, or N > 2^20) every score is stored: per slot
 *    the head-summed query, a histogram, counters, 4 bytes per entry and two candidate lists.
 */
size_t csah_index_topk_workspace(int B, int Q, int64_t N, int k, int HI, int dI);
int csah_index_topk(const uint8_t* q_codes, const uint8_t* q_scales, int HI, int dI,
                    const uint8_t* k_codes, const uint8_t* k_scales, int64_t k_seq_stride,
                    int64_t N, const int64_t* pos, int m, int B, int Q, int k, int32_t* idx_out,
                    float* score_out, void* ws, size_t ws_bytes, void* stream);

/*
 * csah_csa_attend -- sparse attention of every query head over its selected compressed entries,
 * the sliding window of recent uncompressed tokens and a per-head sink, in one softmax.
 *   [EXPL]: each query attends to its top-k compressed entries plus a small window of recent
 *   uncompressed tokens, and an attention-sink term lets a head's weights total less than one;
 *   K and V share one row per entry (shared-KV multi-query layout). [LLMB] "1. CSA": the window
 *   covers the nearest 128 tokens, uncompressed.
 *     s_j = scale * q_h . y_j over rows j in S = {cache row idx[..]} U {window rows},
 *     M = max(sigma_h, max s), den = e^(sigma_h - M) + sum e^(s_j - M),
 *     out_h = sum e^(s_j - M) y_j / den,   lse_h = M + ln(den).
 *   Window rows of query i are rows i .. i+w-1 of the window buffer whose position
 *   pos[b] - (w-1) + r is >= 0 (the w tokens ending at the query's own position).
 *   With sink == NULL the sigma term is absent; an empty row set then gives out = 0, lse = -inf.
 * q         [B][Q][H][D] of q_dtype (CSAH_DT_BF16 or CSAH_DT_F32).
 * cache     [B][cache_seq_stride] rows of fmt (ROW_E4M3_BF16 or ROW_F32), N rows valid.
 * idx       [B][Q][k] int32 entry ids, -1 = empty slot (ids outside [0, N) are skipped too).
 * win       [B][win_seq_stride] rows of fmt; win_seq_stride >= w-1+Q. w may be 0 (win unused).
 * pos       [B] int64 device array, position of query 0.
 * sink      [H] fp32 logits or NULL. scale: softmax temperature applied to q.y.
 * out       [B][Q][H][D] fp32; lse [B][Q][H] fp32 or NULL.
 * ws        at least csah_attend_workspace(B, Q, H, D, k + w) bytes, 256-byte aligned.
 * Supported: any H >= 1 (heads go in groups of 16 per wavefront; the heads that pad the last
 *   group are computed and not stored); (fmt, D) = (ROW_E4M3_BF16, 512) or (ROW_F32, 128);
 *   k + w < 2^31.
 */
size_t csah_attend_workspace(int B, int Q, int H, int D, int64_t max_rows);
int csah_csa_attend(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                    int64_t cache_seq_stride, int64_t N, const int32_t* idx, int k,
                    const void* win, int64_t win_seq_stride, int w, const int64_t* pos,
                    const float* sink, float scale, int B, int Q, float* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * csah_hca_attend -- dense attention over every visible compressed entry plus the same window and
 * sink as csah_csa_attend.
 *   [EXPL]: HCA is the same design with a much larger group and no sparse selection stage, with
 *   the same sliding window and shared-KV layout; [LLMB] "2. HCA": dense attention over the
 *   128x-compressed entries. Query i of sequence b attends to entries g < min(floor((pos[b]+i+1)/m),
 *   N), then to its window rows and the sink exactly as in csah_csa_attend.
 * ws        at least csah_attend_workspace(B, Q, H, D, N + w) bytes, 256-byte aligned.
 * Supported: as csah_csa_attend; m >= 1; N + w < 2^31.
 */
/*
 * csah_csa_attend_noalloc -- csah_csa_attend for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). It takes
 * no workspace: the split partials go to a scratch array of CSAH_NOALLOC_SCRATCH_BYTES (32 MiB)
 * that the library holds in every GPU it runs on until the process ends, so the call neither
 * allocates nor frees anything. Same arguments, layouts, results and statuses as csah_csa_attend
 * without ws / ws_bytes, plus CSAH_ERR_SCRATCH_LIMIT (nothing enqueued) when
 * csah_attend_workspace(B, Q, H, D, k + w) exceeds the scratch; 16 sequences of one query at
 * H = 64, D = 512, k = 1024, w = 128 need 25.4 MB. Every call on a GPU shares that GPU's scratch
 * and nothing in it needs clearing (each call writes every partial it reads); calls that overlap
 * on one GPU (on different streams, or from different threads) race on it and must be ordered by
 * the caller. The first call on a device looks up the scratch's address there.
 */
#define CSAH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int csah_csa_attend_noalloc(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                            int64_t cache_seq_stride, int64_t N, const int32_t* idx, int k,
                            const void* win, int64_t win_seq_stride, int w, const int64_t* pos,
                            const float* sink, float scale, int B, int Q, float* out, float* lse,
                            void* stream);

int csah_hca_attend(const void* q, int q_dtype, int H, int D, const void* cache, int fmt,
                    int64_t cache_seq_stride, int64_t N, int m, const void* win,
                    int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                    float scale, int B, int Q, float* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * Paged caches. A serving system keeps each compressed cache in a pool of fixed-size pages and
 * gives every sequence a block table of page numbers, so that sequences grow without moving rows
 * and memory is handed out page by page. The pages speak of the cache only in general terms
 * (Baidu "Technical Analysis of DeepSeek V4 ...", "Engineering Optimizations": the KV cache is
 * moved in pages; Baidu "Technical Breakdown of DeepSeek V4 Preview ...", "Hardware-Software
 * Co-Optimization": the cache is cut into fixed-size chunks; [BSWEN] "What's Still Missing":
 * inference frameworks must be adapted to the compressed caches). The layout below is this
 * library's own:
 *   pool         rows of the cache's format, page p holding rows [p*P, (p+1)*P) (P = page_size
 *                entries, a power of two in [1, 2^20]). FP4 keys have a second pool of scale
 *                bytes indexed by the same rows.
 *   block_table  int32 [B][table_stride], 4-byte aligned: entry e of sequence b is row
 *                block_table[b*table_stride + e/P] * P + e%P of the pool.
 * Entries keep their LOGICAL numbers everywhere else: top-k indices, visibility, N. Each call
 * computes exactly what its contiguous counterpart computes on the cache gathered back to logical
 * order; only the addressing differs, so the results are bit-identical to that call's.
 * Errors, beyond those of the contiguous call: CSAH_ERR_INVALID_ARGUMENT for a null or misaligned
 * block_table, a page_size that is not a power of two, or a table_stride * P below the entries the
 * call addresses; CSAH_ERR_UNSUPPORTED for page_size > 2^20. Table entries are device data: each
 * one a call reads (the pages of entries [0, N), or of the entries written) must name a page that
 * lies inside the pool; the library cannot check this.
 */

/*
 * csah_kv_compress_paged -- csah_kv_compress_span writing its entries into a paged cache: output
 * entry g of sequence b (g in [0, T/m - skip)) goes to logical entry first_entry + g of that
 * sequence. out_pool / out_scale_pool as out_rows / out_scales. first_entry >= 0 and
 * (first_entry + T/m - skip) <= table_stride * page_size.
 */
int csah_kv_compress_paged(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                           int64_t T, int D, int m, int span, int64_t skip, const float* w,
                           const float* beta, void* out_pool, int out_fmt,
                           uint8_t* out_scale_pool, const int32_t* block_table,
                           int64_t table_stride, int page_size, int64_t first_entry,
                           void* stream);

/*
 * csah_index_topk_paged -- csah_index_topk over FP4 keys held in a paged pool (codes and scales
 * pools share the block table). table_stride * page_size >= N. Indices are logical entry numbers.
 * Workspace as csah_index_topk_workspace(B, Q, N, k, HI, dI).
 */
int csah_index_topk_paged(const uint8_t* q_codes, const uint8_t* q_scales, int HI, int dI,
                          const uint8_t* k_pool_codes, const uint8_t* k_pool_scales,
                          const int32_t* block_table, int64_t table_stride, int page_size,
                          int64_t N, const int64_t* pos, int m, int B, int Q, int k,
                          int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * csah_csa_attend_paged / csah_hca_attend_paged -- csah_csa_attend / csah_hca_attend with the
 * compressed cache in a paged pool; idx holds logical entry numbers. The window buffer stays a
 * per-sequence array as in the contiguous calls. table_stride * page_size >= N.
 */
int csah_csa_attend_paged(const void* q, int q_dtype, int H, int D, const void* cache_pool,
                          int fmt, const int32_t* block_table, int64_t table_stride,
                          int page_size, int64_t N, const int32_t* idx, int k, const void* win,
                          int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                          float scale, int B, int Q, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream);
int csah_hca_attend_paged(const void* q, int q_dtype, int H, int D, const void* cache_pool,
                          int fmt, const int32_t* block_table, int64_t table_stride,
                          int page_size, int64_t N, int m, const void* win,
                          int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                          float scale, int B, int Q, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * RoPE on the rotary dims.
 *   [BSWEN] "Component 1: Shared Key-Value Vectors": keys and values are one shared vector, and an
 *   inverse RoPE restores its positional information; [EXPL] "Key numbers" (KV storage precision
 *   row): a row's rotary dims are its BF16 part. The pages define neither the rotation nor its
 *   frequencies; the library uses RoFormer's general form (Su et al., "RoFormer: Enhanced
 *   Transformer with Rotary Position Embedding", section 3.2): the LAST R = rope_dims dims of a
 *   D-wide row form R/2 adjacent pairs (2j, 2j+1), and at position p pair j turns
 *   counter-clockwise by p * theta_j, theta_j = rope_base^(-2j/R):
 *     (a, b) -> (a cos - b sin, a sin + b cos);   the inverse turns back by the same angle.
 *   Angles, sines and cosines are computed in fp64, so positions of 2^20 and beyond keep their
 *   accuracy. The use on the path: queries are turned at their positions before attention, each
 *   compressed entry when it is written (csah_kv_compress_rope), and the attention output is
 *   turned back at the query's position (inverse), which leaves every value's rotary part turned
 *   by the entry's position relative to the query.
 *   Constraints: D even, R even, 2 <= R <= D, rope_base finite and > 0, else
 *   CSAH_ERR_INVALID_ARGUMENT.
 */

/*
 * csah_rope -- turn the rotary dims of rows x [B][Q][H][D] in place. Row group (b, i) (all H
 * heads) sits at position pos[b] + i (the queries' position rule of every call above).
 * x         device array of dtype CSAH_DT_BF16 or CSAH_DT_F32, 16-byte aligned, contiguous.
 *           bf16 rows are rounded once from the fp64 result (nearest, ties to even), f32 rows
 *           likewise. Dims before D - R are not read or written.
 * pos       [B] int64 device array, 8-byte aligned.
 * inverse   0: turn forward; 1: turn back (the inverse RoPE of the attention output).
 * Returns CSAH_OK without touching anything when B = 0 or Q = 0; CSAH_ERR_UNSUPPORTED for
 * R > 1024, B*Q > 2^31 - 1 or H*R > 2^28.
 */
int csah_rope(void* x, int dtype, int B, int Q, int H, int D, int rope_dims, const int64_t* pos,
              double rope_base, int inverse, void* stream);

/*
 * csah_kv_compress_rope -- csah_kv_compress_span whose pooled entries are turned by RoPE before
 * they are encoded. The entry of group g of raw (g counted from raw's token 0, context groups
 * included) sits at the position of the group's last token, tok_pos[b] + m(g+1) - 1: the token
 * that completes the group and makes the entry visible, whatever the span.
 * tok_pos   [B] int64 device array (8-byte aligned): position of raw's token 0 of each sequence.
 * rope_dims must be nonzero; other arguments and statuses as csah_kv_compress_span.
 */
int csah_kv_compress_rope(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                          int64_t T, int D, int m, int span, int64_t skip, const float* w,
                          const float* beta, void* out_rows, int out_fmt, int64_t out_seq_stride,
                          uint8_t* out_scales, const int64_t* tok_pos, int rope_dims,
                          double rope_base, void* stream);

/*
 * csah_kv_compress_paged_rope -- csah_kv_compress_paged with the RoPE of csah_kv_compress_rope.
 */
int csah_kv_compress_paged_rope(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                                int64_t T, int D, int m, int span, int64_t skip, const float* w,
                                const float* beta, void* out_pool, int out_fmt,
                                uint8_t* out_scale_pool, const int32_t* block_table,
                                int64_t table_stride, int page_size, int64_t first_entry,
                                const int64_t* tok_pos, int rope_dims, double rope_base,
                                void* stream);

/*
 * csah_profile_next_call -- profiling aid (not part of the method). The next compression,
 * indexer, attention or RoPE call (any of the calls above) made by the SAME host thread launches
 * its dominant kernel (the compressor; the indexer scan; the attention kernel; the rotation) with `begin` and
 * `end` attached to that dispatch, so that hipEventElapsedTime(begin, end) is the kernel's own
 * duration. Both are hipEvent_t passed as void*, created by the caller with timing enabled; NULL
 * for both cancels a pending request. The request is consumed by that
 * next call whether or not it succeeds. Returns CSAH_OK, or CSAH_ERR_INVALID_ARGUMENT if exactly
 * one event is NULL.
 */
int csah_profile_next_call(void* begin_event, void* end_event);

#ifdef __cplusplus
}
#endif

#endif /* CSAH_H */
