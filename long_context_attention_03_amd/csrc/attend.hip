// attend.hip -- sparse (CSA) and dense (HCA) attention over shared K=V rows, window and sink.
//
// [EXPL] "DeepSeek V4 Architecture Explained: CSA, HCA, mHC and Muon", section "How
// compress-then-sparsify attention works": each query attends to its top-k compressed entries, a
// sliding window of recent uncompressed tokens keeps local fidelity, and an attention-sink term lets
// a head's weights total less than one; HCA attends to all compressed entries with the same window
// and sink, and both use a shared-KV multi-query layout (one K=V row serves every head).
// [LLMB] "Inside DeepSeek-V4 ...", sections "1. CSA" (window of the nearest 128 tokens) and
// "2. HCA" (dense attention over the compressed entries).
//
// One softmax covers compressed rows, window rows and the sink:
//   out_h = sum_j e^(s_j - M) y_j / (e^(sigma_h - M) + sum_j e^(s_j - M)),  s_j = scale q_h . y_j.
//
// Mapping onto gfx950. All H heads of a query share every row, so per row block the work is a dense
// contraction with 16 heads per wavefront: S^T = Y Q^T (rows x heads, K = D) and
// O^T += Y^T P^T (D x heads, K = rows), both on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//   - Y (E4M3 + bf16 rows) converts exactly to bf16, so Q.Y products are exact; fp32 rows are split
//     into hi + lo bf16 terms. P in (0, 1] is split into hi + lo bf16 terms (about 16 significant
//     bits), so the PV contraction keeps fp32-level accuracy.
//   - The QK A-operand is loaded straight from HBM (lane l: row l%16, 8 dims at 8*(l/16)) and
//     converted in registers; the same bf16 fragments are stored row-major into a per-wavefront
//     LDS tile (one 16-byte write each, rows padded by 32 bytes). The PV A-operand Y^T is read
//     back with gfx950's transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group,
//     output lane n, element e comes from input lane 4e + n/4, element n%4, so lane (e, q) of
//     group g points at row 4g+e (then 16+4g+e), dims 16t+4q, and receives dim 16t+n of those
//     four rows. The K-slot order this produces matches the C layout of S^T, so P never moves
//     between lanes.
//   - The next tile's row loads are issued as soon as the QK phase has consumed the registers, so
//     they overlap the softmax and PV phase.
//   - Online softmax in base 2 with a lazily updated reference max per head: the accumulators are
//     rescaled only when a head's max grows by more than 2^8 (P <= 256 otherwise).
// Grid: one workgroup per (sequence x query, row split, head group of 16), mapped XCD-aware. The 4 wavefronts of a workgroup take
// 32-row tiles of the split in turn and are merged in LDS at the end; with one split the workgroup
// applies the sink and writes the output, otherwise it writes (max, sum, acc) partials that
// attend_merge_kernel combines with the sink.
#include "csah_internal.h"
#include "device_common.h"

namespace csah {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int kTile = 32;   // rows per wavefront tile
constexpr int kWaves = 4;

template <int FMT>
struct RowCfg;
template <>
struct RowCfg<CSAH_FMT_ROW_E4M3_BF16> {
  static constexpr int D = 512, NCH = 16, YS = 1, RB = 576;
};
template <>
struct RowCfg<CSAH_FMT_ROW_F32> {
  static constexpr int D = 128, NCH = 4, YS = 2, RB = 512;
};

struct AttendK {
  const void* q;
  int H;
  const uint8_t* cache;
  EntryMap cmap;  // entry e of sequence b is row cmap.row(b, e) of `cache`
  int64_t N;
  const int32_t* idx;
  int k, m;
  const uint8_t* win;
  int64_t wstride;
  int w;
  const int64_t* pos;
  const float* sink;
  float scale_log2;
  int Q, splits, rows_per_split, hg, slots;
  float* out;
  float* lse;
  float* part;
};

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; e++) r[e] = (__bf16)x[e];
  return r;
}

// Raw register image of one lane's share of a 32-row tile: rows n and 16+n, dims [32c+8g, +8)
// of every 32-wide chunk c. Loaded unconditionally (masked rows read a valid dummy row) so that a
// whole tile's loads are in flight together and never wait inside a branch.
template <int FMT>
struct TileRaw;
template <>
struct TileRaw<CSAH_FMT_ROW_E4M3_BF16> {
  u32x2 e[2][14];  // E4M3 bytes of dims 32c+8g.. (c < 14)
  u32x4 r[2][2];   // bf16 rotary dims 448+32(c-14)+8g..
};
template <>
struct TileRaw<CSAH_FMT_ROW_F32> {
  f32x4 v[2][4][2];
};

template <int FMT>
__device__ __forceinline__ void load_tile(const uint8_t* p0, const uint8_t* p1, int g,
                                          TileRaw<FMT>& t) {
  const uint8_t* ps[2] = {p0, p1};
#pragma unroll
  for (int r = 0; r < 2; r++) {
    if constexpr (FMT == CSAH_FMT_ROW_E4M3_BF16) {
#pragma unroll
      for (int c = 0; c < 14; c++) t.e[r][c] = *(const u32x2*)(ps[r] + 32 * c + 8 * g);
#pragma unroll
      for (int c = 0; c < 2; c++) t.r[r][c] = *(const u32x4*)(ps[r] + 448 + 64 * c + 16 * g);
    } else {
#pragma unroll
      for (int c = 0; c < 4; c++) {
        t.v[r][c][0] = *(const f32x4*)(ps[r] + 4 * (32 * c + 8 * g));
        t.v[r][c][1] = *(const f32x4*)(ps[r] + 4 * (32 * c + 8 * g) + 16);
      }
    }
  }
}

// bf16 fragment (hi, and lo for fp32 rows) of row r, chunk c; zero when the row is masked.
template <int FMT>
__device__ __forceinline__ void tile_frag(const TileRaw<FMT>& t, int r, int c, bool valid,
                                          bf16x8& hi, bf16x8& lo) {
  if constexpr (FMT == CSAH_FMT_ROW_E4M3_BF16) {
    if (c < 14) {
      const u32x2 v = t.e[r][c];
      const uint32_t w0 = valid ? v[0] : 0u, w1 = valid ? v[1] : 0u;
      bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
      bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
      bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
      bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
      hi = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    } else {
      u32x4 v = t.r[r][c - 14];
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = valid ? v[e] : 0u;
      hi = __builtin_bit_cast(bf16x8, v);
    }
  } else {
    const f32x4 a = t.v[r][c][0], b = t.v[r][c][1];
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    float rr[8];
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = valid ? x[e] : 0.0f;
    hi = pack_bf16x8(x);
#pragma unroll
    for (int e = 0; e < 8; e++) rr[e] = x[e] - (float)hi[e];
    lo = pack_bf16x8(rr);
  }
}

template <int FMT, int QDT, bool DENSE>
__global__ __launch_bounds__(256, 1) void attend_kernel(AttendK p) {
  using C = RowCfg<FMT>;
  constexpr int D = C::D, NCH = C::NCH, YS = C::YS, NT = D / 16;
  constexpr int QS = QDT == CSAH_DT_F32 ? 2 : 1;
  constexpr int RS = D + 16;                    // LDS row stride (bf16 elements)
  constexpr int YT_ELEMS = kTile * RS;          // bf16 elements per wavefront per split term
  constexpr int LDS_YT = kWaves * YS * YT_ELEMS * 2;
  constexpr int LDS_COMB = kWaves * 16 * D * 4;
  constexpr int LDS_BYTES = LDS_YT > LDS_COMB ? LDS_YT : LDS_COMB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  __shared__ float s_ml[kWaves][16][2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8). Consecutive workgroups of one
  // XCD take the head groups of one (query, split) unit, so the rows they all read are fetched
  // into that XCD's L2 once.
  const int64_t wg = blockIdx.x;
  const int64_t unit = (wg / (8 * p.hg)) * 8 + (wg & 7);
  const int hgi = (int)((wg >> 3) % p.hg);
  if (unit >= (int64_t)p.splits * p.slots) return;
  const int slot = (int)(unit / p.splits), split = (int)(unit - (int64_t)slot * p.splits);
  const int b = slot / p.Q, qi = slot - b * p.Q;

  // ---- query fragments: B operand of S^T = Y Q^T (k = dims 32c + 8g + e, n = head) ----
  bf16x8 qf[QS][NCH];
  {
    const int head = hgi * 16 + n;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      float x[8];
      if (head < p.H) {
        const int64_t qo = ((int64_t)slot * p.H + head) * D + 32 * c + 8 * g;
        if constexpr (QDT == CSAH_DT_BF16) {
          qf[0][c] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const uint16_t*)p.q + qo));
          continue;
        } else {
          const float* qp = (const float*)p.q + qo;
          const f32x4 a = *(const f32x4*)qp, bb = *(const f32x4*)(qp + 4);
          x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
          x[4] = bb[0]; x[5] = bb[1]; x[6] = bb[2]; x[7] = bb[3];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = 0.0f;
      }
      qf[0][c] = pack_bf16x8(x);
      if constexpr (QS == 2) {
        float r8[8];
#pragma unroll
        for (int e = 0; e < 8; e++) r8[e] = x[e] - (float)qf[0][c][e];
        qf[QS - 1][c] = pack_bf16x8(r8);
      }
    }
  }

  // ---- the logical row range of this split ----
  const int64_t pos_b = p.pos[b];
  int64_t Rc;
  if constexpr (DENSE) {
    int64_t nv = (pos_b + qi + 1) / p.m;
    Rc = nv < 0 ? 0 : (nv > p.N ? p.N : nv);
  } else {
    Rc = p.N > 0 ? p.k : 0;  // no compressed row can be valid without entries: none is read
  }
  const int64_t R = Rc + p.w;
  const int64_t r0 = (int64_t)split * p.rows_per_split;
  const int64_t r1 = r0 + p.rows_per_split < R ? r0 + p.rows_per_split : R;
  const int64_t rc_end = Rc < r1 ? Rc : r1;  // compressed rows of this split end here
  // a readable row for masked slots (a tile with any valid row implies N > 0 or w > 0)
  const uint8_t* dummy = p.N > 0 ? p.cache + p.cmap.row(b, 0) * C::RB
                                 : p.win + (int64_t)b * p.wstride * C::RB;

  // entry id of tile row (lane & 31), fetched one tile ahead of its use (CSA only)
  auto fetch_idx = [&](int64_t t) -> int32_t {
    if constexpr (DENSE) {
      return 0;
    } else {
      if (p.k == 0) return -1;
      int64_t j = t + (lane & 31);
      j = j < Rc ? j : Rc - 1;
      j = j < 0 ? 0 : j;
      return p.idx[(int64_t)slot * p.k + j];
    }
  };
  // row j -> (pointer, valid); e = entry id for CSA rows
  auto resolve = [&](int64_t j, int32_t e, bool& valid) -> const uint8_t* {
    const uint8_t* ptr = dummy;
    valid = false;
    if (j < rc_end) {
      const int64_t ent = DENSE ? j : (int64_t)e;
      if (ent >= 0 && ent < p.N) {
        valid = true;
        ptr = p.cache + p.cmap.row(b, ent) * C::RB;
      }
    } else if (j < r1) {
      const int64_t r = qi + (j - Rc);              // window buffer row
      if (pos_b - (p.w - 1) + r >= 0) {             // its token position is >= 0
        valid = true;
        ptr = p.win + ((int64_t)b * p.wstride + r) * C::RB;
      }
    }
    return ptr;
  };
  // pointers of rows n and 16+n, the tile's validity mask, and the loads of its rows
  auto prep_tile = [&](int64_t t, int32_t e_lane, TileRaw<FMT>& raw, uint32_t& mask) {
    bool vm;
    (void)resolve(t + (lane & 31), e_lane, vm);
    mask = (uint32_t)ballot64(vm);
    const int32_t e0 = __shfl(e_lane, n, 64), e1 = __shfl(e_lane, 16 + n, 64);
    bool v0, v1;
    const uint8_t* p0 = resolve(t + n, e0, v0);
    const uint8_t* p1 = resolve(t + 16 + n, e1, v1);
    load_tile<FMT>(p0, p1, g, raw);
  };

  // per-wavefront row-major bf16 tile: Y[row][RS]
  __bf16* yt = (__bf16*)smem + wave * YS * YT_ELEMS;
  // transposing-read base: lane (e, q) of group g reads row 4g+e, dims 4q.. (+16t per d-tile)
  const int tr_row = 4 * g + ((lane & 15) >> 2), tr_col = 4 * (lane & 3);
  typedef __attribute__((address_space(3))) short4_t* lds_s4_ptr;
  f32x4 O[NT];
#pragma unroll
  for (int t = 0; t < NT; t++) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  constexpr int64_t kStep = (int64_t)kTile * kWaves;

  int64_t tb = r0 + (int64_t)kTile * wave;
  TileRaw<FMT> raw;
  uint32_t mask_cur = 0;
  int32_t e_next = 0;
  if (tb < r1) {
    const int32_t e0 = fetch_idx(tb);
    e_next = fetch_idx(tb + kStep);
    prep_tile(tb, e0, raw, mask_cur);
  }
  for (; tb < r1; tb += kStep) {
    const uint32_t mask = mask_cur;
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
    f32x4 S0b = {0.f, 0.f, 0.f, 0.f}, S1b = {0.f, 0.f, 0.f, 0.f};  // odd chunks: shorter chains
    if (mask != 0u) {
      const bool v0 = (mask >> n) & 1u, v1 = (mask >> (16 + n)) & 1u;
      // S^T for rows tb..tb+15 (S0) and tb+16..tb+31 (S1); stage Y row-major in LDS
#pragma unroll
      for (int c = 0; c < NCH; c++) {
        bf16x8 a0h, a0l, a1h, a1l;
        tile_frag<FMT>(raw, 0, c, v0, a0h, a0l);
        tile_frag<FMT>(raw, 1, c, v1, a1h, a1l);
        f32x4& A0 = (c & 1) ? S0b : S0;
        f32x4& A1 = (c & 1) ? S1b : S1;
        A0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0h, qf[0][c], A0, 0, 0, 0);
        A1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1h, qf[0][c], A1, 0, 0, 0);
        if constexpr (QS == 2) {
          A0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0h, qf[1][c], A0, 0, 0, 0);
          A1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1h, qf[1][c], A1, 0, 0, 0);
        }
        if constexpr (YS == 2) {
          A0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0l, qf[0][c], A0, 0, 0, 0);
          A1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1l, qf[0][c], A1, 0, 0, 0);
        }
        *(bf16x8*)(yt + n * RS + 32 * c + 8 * g) = a0h;
        *(bf16x8*)(yt + (16 + n) * RS + 32 * c + 8 * g) = a1h;
        if constexpr (YS == 2) {
          *(bf16x8*)(yt + YT_ELEMS + n * RS + 32 * c + 8 * g) = a0l;
          *(bf16x8*)(yt + YT_ELEMS + (16 + n) * RS + 32 * c + 8 * g) = a1l;
        }
      }
    }
    S0 += S0b;
    S1 += S1b;
    // the row registers are free: start the next tile's loads (and the ids of the one after)
    uint32_t mask_nxt = 0;
    if (tb + kStep < r1) {
      const int32_t e_after = fetch_idx(tb + 2 * kStep);
      prep_tile(tb + kStep, e_next, raw, mask_nxt);
      e_next = e_after;
    }
    if (mask != 0u) {
      // online softmax (base 2); lane holds rows 4g+i (S0) and 16+4g+i (S1) of head n
      float v[8];
      if (mask == 0xFFFFFFFFu) {  // every row valid (all but the edge tiles)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          v[i] = S0[i] * p.scale_log2;
          v[4 + i] = S1[i] * p.scale_log2;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          v[i] = ((mask >> (4 * g + i)) & 1u) ? S0[i] * p.scale_log2 : -INFINITY;
          v[4 + i] = ((mask >> (16 + 4 * g + i)) & 1u) ? S1[i] * p.scale_log2 : -INFINITY;
        }
      }
      float tmax = v[0];
#pragma unroll
      for (int i = 1; i < 8; i++) tmax = fmaxf(tmax, v[i]);
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      // lazy rescale: the reference max moves only when a head's max grows by more than 2^8, so
      // P stays below 256 and the accumulators are rescaled rarely
      const float m_new = fmaxf(m_run, tmax);
      if (__ballot(m_new > m_run + 8.0f)) {
        const float alpha = exp2f(m_run - m_new);  // 0 while nothing was accumulated
        if (__ballot(m_run != -INFINITY && alpha != 1.0f)) {
#pragma unroll
          for (int t = 0; t < NT; t++) O[t] *= alpha;
        }
        l_run *= alpha;
        m_run = m_new;
      }
      float P[8], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        P[i] = __builtin_amdgcn_exp2f(v[i] - m_run);  // v - m_run <= 8; -inf gives 0
        psum += P[i];
      }
      l_run += psum;
      bf16x8 ph, pl;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        ph[e] = (__bf16)P[e];
        pl[e] = (__bf16)(P[e] - (float)ph[e]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // O^T += Y^T P^T, Y^T fragments by transposing reads of the row-major tile
      auto ytr = [&](int t, int term) -> bf16x8 {
        const __bf16* base0 = yt + term * YT_ELEMS + tr_row * RS + 16 * t + tr_col;
        const short4_t y0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)base0);
        const short4_t y1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(base0 + 16 * RS));
        return __builtin_bit_cast(
            bf16x8, short8_t{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]});
      };
      // two d-tiles at a time so that dependent accumulations are never back to back
#pragma unroll
      for (int t = 0; t < NT; t += 2) {
        const bf16x8 ya = ytr(t, 0), yb = ytr(t + 1, 0);
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ya, ph, O[t], 0, 0, 0);
        O[t + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yb, ph, O[t + 1], 0, 0, 0);
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ya, pl, O[t], 0, 0, 0);
        O[t + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yb, pl, O[t + 1], 0, 0, 0);
        if constexpr (YS == 2) {
          const bf16x8 za = ytr(t, 1), zb = ytr(t + 1, 1);
          O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, ph, O[t], 0, 0, 0);
          O[t + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zb, ph, O[t + 1], 0, 0, 0);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    mask_cur = mask_nxt;
  }

  // ---- merge the 4 wavefronts ----
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  constexpr int CS = D + 4;  // padded row: the 16 heads of one wave land in different banks
  static_assert(kWaves * 16 * CS * 4 <= LDS_BYTES, "merge buffer fits the tile buffers");
  __syncthreads();
  float* comb = (float*)smem;  // [wave][16 heads][CS]
#pragma unroll
  for (int t = 0; t < NT; t++)
    *(f32x4*)(comb + (wave * 16 + n) * CS + 16 * t + 4 * g) = O[t];
  if (g == 0) {
    s_ml[wave][n][0] = m_run;
    s_ml[wave][n][1] = l_run;
  }
  __syncthreads();
  // per head: M = max over waves, weights 2^(m_w - M), L = sum of weighted sums (64 threads)
  __shared__ float s_wgt[kWaves][16];
  __shared__ float s_hm[16][2];
  if (threadIdx.x < 16) {
    const int hl = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; wv++) M = fmaxf(M, s_ml[wv][hl][0]);
    float L = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; wv++) {
      const float mw = s_ml[wv][hl][0];
      const float om = mw == -INFINITY ? 0.0f : exp2f(mw - M);
      s_wgt[wv][hl] = om;
      L = fmaf(s_ml[wv][hl][1], om, L);
    }
    const int hh = hgi * 16 + hl;
    if (p.splits == 1) {
      float Mf = M, den = L, a = 1.0f;
      if (p.sink && hh < p.H) {
        const float sg = p.sink[hh] * kLog2e;
        Mf = fmaxf(M, sg);
        a = M == -INFINITY ? 0.0f : exp2f(M - Mf);
        den = L * a + exp2f(sg - Mf);
      }
      s_hm[hl][0] = den > 0.0f ? a / den : 0.0f;  // output scale
      if (p.lse && hh < p.H)
        p.lse[(int64_t)slot * p.H + hh] = den > 0.0f ? (Mf + log2f(den)) * kLn2 : -INFINITY;
    } else {
      s_hm[hl][0] = M;
      s_hm[hl][1] = L;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += 256) {
    const int hl = e / D, d = e - hl * D;
    const int hh = hgi * 16 + hl;
    if (hh >= p.H) continue;
    float acc = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; wv++) acc = fmaf(comb[(wv * 16 + hl) * CS + d], s_wgt[wv][hl], acc);
    if (p.splits == 1) {
      p.out[((int64_t)slot * p.H + hh) * D + d] = acc * s_hm[hl][0];
    } else {
      // partial row: acc[D], max, sum, 2 pad floats (16-byte aligned rows)
      float* pp = p.part + (((int64_t)slot * p.splits + split) * p.H + hh) * (D + 4);
      pp[d] = acc;
      if (d == 0) {
        pp[D] = s_hm[hl][0];
        pp[D + 1] = s_hm[hl][1];
      }
    }
  }
}

// ================================================================================================
// E4M3 + bf16 rows (D = 512) with bf16 queries: workgroups that share converted row tiles.
//
// A workgroup of 4 wavefronts owns one (query, row split, block of 64 heads); wavefront w takes
// head group w (16 heads). The 256 threads load each 32-row tile once: thread t takes row t/8,
// bytes 64i+8(t%8) (i < 7) of the E4M3 part and 448+16(t%8) of the bf16 part, so every load
// instruction reads 64 contiguous bytes per row. The tile is converted exactly to bf16 and stored
// row-major (1056-byte LDS rows, the stride measured conflict-free for both read patterns) in a
// double-buffered tile that the four head groups share: 16-byte reads give the A-fragments of
// S^T = Y Q^T, the transposing read gives the Y^T fragments of O^T += Y^T P^T, as in
// attend_kernel. One workgroup barrier per tile orders the buffer reuse (a buffer is rewritten two
// tiles later, after every wavefront has passed the barrier of the tile in between). The next
// tile's loads are issued after the S^T phase and land during the softmax and P.Y phases. With
// MINW = 2 two workgroups share a CU (LDS 67.6 KB, at most 256 registers per lane each), so one's
// barrier and softmax waits overlap the other's matrix work; with MINW = 1 a workgroup keeps more
// tiles in flight instead.
constexpr int kXTile = 32, kXRS = 528, kXTileElems = kXTile * kXRS;
// a tile's lo term is left out when its largest weight is at most this share of the lane's sum
constexpr float kLoSkipFrac = 0.0625f;

// Max over the four 16-lane rows of a wavefront, in every lane: gfx950's permlane swaps exchange
// rows 0<->1 and 2<->3 (16-lane swap), then the two halves (32-lane swap), so each lane ends up
// holding the max of lanes l, l^16, l^32 and l^48.
__device__ __forceinline__ float max_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  x = fmaxf(u2f(a[0]), u2f(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(c[0]), u2f(c[1]));
}

struct TileRawX {
  u32x2 e[7];  // E4M3 bytes 64i + 8(t%8) .. +8
  u32x4 r;     // bf16 dims 448 + 8(t%8) .. +8
};

// MINW: workgroups per CU the register budget is sized for. Grids of up to one workgroup per CU
// (decode) take 1, so a wavefront may hold all 512 registers and nothing spills; larger grids
// (prefill) take 2, so two workgroups overlap each other's waits.
// SKIPLO (two-per-CU build, splits of 64 tiles or more): tiles whose weights are all small next to
// the weight already summed leave out the lo term of P (see the softmax below). Shorter splits
// seldom reach that state and run faster with the hi and lo products interleaved.
template <bool DENSE, bool PAGED, int MINW, bool SKIPLO>
__global__ __launch_bounds__(256, MINW) void attend_x_kernel(AttendK p) {
  constexpr int D = 512, NCH = 16, NT = 32, RB = 576;
  // Tiles whose rows are in flight: with a CU's whole register file (MINW = 1) the rows of the
  // next two tiles load while one is computed, which covers a gather's latency; with two
  // workgroups per CU the other workgroup covers it and one tile ahead keeps registers free.
  constexpr int PREF = MINW == 1 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) __bf16 ytile[2][kXTileElems];  // double buffer
  __shared__ uint32_t s_mask[2][4];  // [buffer][loading wavefront]: 8 row bits each

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hgl = wave;  // head group
  const int g = lane >> 4, n = lane & 15;
  const int lrow = tid >> 3, lk = tid & 7;  // the tile row this thread loads, its slot
  // Workgroups are dispatched round-robin over the 8 XCDs; consecutive workgroups of one XCD take
  // the head blocks of one (query, split) unit so that its rows are fetched into one L2.
  // (32-bit workgroup arithmetic, kept in scalar registers: grids stay below 2^31)
  // Every kernel argument in one round trip: left alone, the compiler loads each field where it
  // is first used, and the chain of dependent scalar loads costs microseconds at start-up.
  asm volatile("" ::"s"(p.q), "s"(p.H), "s"(p.cache), "s"(p.cmap.table), "s"(p.cmap.stride),
               "s"(p.cmap.shift), "s"(p.N), "s"(p.idx), "s"(p.k), "s"(p.m), "s"(p.win),
               "s"(p.wstride), "s"(p.w), "s"(p.pos), "s"(p.sink), "s"(p.scale_log2), "s"(p.Q),
               "s"(p.splits), "s"(p.rows_per_split), "s"(p.hg), "s"(p.slots), "s"(p.out),
               "s"(p.lse), "s"(p.part));
  const int wg = blockIdx.x;
  const int unit = (wg / (8 * p.hg)) * 8 + (wg & 7);
  const int hb = (wg >> 3) % p.hg;
  if (unit >= p.splits * p.slots) return;
  const int slot = __builtin_amdgcn_readfirstlane(unit / p.splits);
  const int split = unit - slot * p.splits;
  const int b = __builtin_amdgcn_readfirstlane(slot / p.Q), qi = slot - b * p.Q;
  const int head = hb * 64 + hgl * 16 + n;

  // the logical rows of this split: compressed rows [0, Rc), then the w window rows
  const int64_t pos_b = p.pos[b];
  int64_t Rc;
  if constexpr (DENSE) {
    int64_t nv = (pos_b + qi + 1) / p.m;
    Rc = nv < 0 ? 0 : (nv > p.N ? p.N : nv);
  } else {
    Rc = p.N > 0 ? p.k : 0;  // no compressed row can be valid without entries: none is read
  }
  const int64_t R = Rc + p.w;
  const int64_t r0 = (int64_t)split * p.rows_per_split;
  const int64_t r1 = r0 + p.rows_per_split < R ? r0 + p.rows_per_split : R;
  const int64_t rc_end = Rc < r1 ? Rc : r1;
  // Every tile issues the same loads whether its rows exist or not (absent rows read a dummy
  // that is always mapped: a cache or window row, else the query), so the wait before a tile's
  // rows are used covers only that tile: a skipped load would make the wait drain every load in
  // flight. Index loads of absent rows read this sequence's position instead.
  const uint8_t* dummy =
      p.N > 0 ? p.cache + (PAGED ? p.cmap.paged(b, 0) : p.cmap.flat(b, 0)) * RB
              : (p.w > 0 ? p.win + (int64_t)b * p.wstride * RB : (const uint8_t*)p.q);
  const int32_t* dummy_i = (const int32_t*)(p.pos + b);
  const int ntiles = r1 > r0 ? (int)((r1 - r0 + kXTile - 1) / kXTile) : 0;
  const int iters = ntiles;

  // entry id of this thread's row in the tile starting at tbase (CSA only)
  auto fetch_id = [&](int64_t tbase) -> int32_t {
    if constexpr (DENSE) {
      return 0;
    } else {
      const int64_t j = tbase + lrow;
      const int32_t e = *(j < rc_end ? p.idx + (int64_t)slot * p.k + j : dummy_i);
      return j < rc_end ? e : -1;
    }
  };
  // Paged caches: a row's pool row comes from the block table, a load that depends on the
  // entry id. Ids are fetched two tiles ahead and translated one tile ahead, so neither load
  // is waited for while the current tile's rows are in flight.
  auto pool_row = [&](int64_t j, int32_t e) -> int64_t {  // -1: not a valid compressed row
    const int64_t ent = DENSE ? j : (int64_t)e;
    const bool ok = j < rc_end && ent >= 0 && ent < p.N;
    if constexpr (PAGED) {
      const int64_t page = *(ok ? p.cmap.table + (int64_t)b * p.cmap.stride + (ent >> p.cmap.shift)
                                : dummy_i);
      return ok ? (page << p.cmap.shift) | (ent & (((int64_t)1 << p.cmap.shift) - 1)) : -1;
    } else {
      return ok ? p.cmap.flat(b, ent) : -1;
    }
  };
  auto resolve_row = [&](int64_t j, int64_t prow, bool& valid) -> const uint8_t* {
    valid = false;
    const uint8_t* ptr = dummy;
    if (j < rc_end) {
      if (prow >= 0) {
        valid = true;
        ptr = p.cache + prow * RB;
      }
    } else if (j < r1) {
      const int64_t r = qi + (j - Rc);
      if (pos_b - (p.w - 1) + r >= 0) {
        valid = true;
        ptr = p.win + ((int64_t)b * p.wstride + r) * RB;
      }
    }
    return ptr;
  };
  auto load_rows = [&](const uint8_t* ptr, TileRawX& t) {
#pragma unroll
    for (int i = 0; i < 7; i++) t.e[i] = *(const u32x2*)(ptr + 64 * i + 8 * lk);
    t.r = *(const u32x4*)(ptr + 448 + 16 * lk);
  };

  const int tr_row = 4 * g + ((lane & 15) >> 2), tr_col = 4 * (lane & 3);
  typedef __attribute__((address_space(3))) short4_t* lds_s4_ptr;
  f32x4 O[NT];
#pragma unroll
  for (int t = 0; t < NT; t++) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // Ring of PREF slots, one per tile in flight. Before iteration it (slot it % PREF) the slot holds
  // the rows of tile it, the pool row of this thread's row of tile it + PREF and the entry id of
  // tile it + 2 PREF: each load is issued a slot cycle before the one that depends on it.
  // Start-up order: every id first (one wait covers them), then the first tile's rows, the query
  // fragments and the other tiles' rows, so that the first tile and the query arrive together
  // and neither waits behind the rest.
  TileRawX raw[PREF];
  bool v_raw[PREF];
  int64_t pr[PREF];
  int32_t ee[PREF], ea[PREF], eb[PREF];
#pragma unroll
  for (int k = 0; k < PREF; k++) {
    const int64_t tk = r0 + (int64_t)k * kXTile;
    ea[k] = fetch_id(tk);
    eb[k] = fetch_id(tk + PREF * kXTile);
    ee[k] = fetch_id(tk + 2 * PREF * kXTile);
  }
  int64_t pa[PREF];
#pragma unroll
  for (int k = 0; k < PREF; k++) pa[k] = pool_row(r0 + (int64_t)k * kXTile + lrow, ea[k]);
  load_rows(resolve_row(r0 + lrow, pa[0], v_raw[0]), raw[0]);
  // query fragments: B operand of S^T = Y Q^T (k = dims 32c + 8g + e, n = head)
  bf16x8 qf[NCH];
  {
    // Heads past H compute with head 0's query: their results are never stored, and nothing
    // mixes heads, so no load sits in a branch and no select waits for the loaded values.
    const uint16_t* qrow =
        (const uint16_t*)p.q + ((int64_t)slot * p.H + (head < p.H ? head : 0)) * D;
#pragma unroll
    for (int c = 0; c < NCH; c++)
      qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * c + 8 * g));
  }
#pragma unroll
  for (int k = 1; k < PREF; k++)
    load_rows(resolve_row(r0 + (int64_t)k * kXTile + lrow, pa[k], v_raw[k]), raw[k]);
#pragma unroll
  for (int k = 0; k < PREF; k++) pr[k] = pool_row(r0 + (int64_t)(k + PREF) * kXTile + lrow, eb[k]);
  // refill a slot once its rows are consumed: rows of tile it + PREF, pool row of tile
  // it + 2 PREF, id of tile it + 3 PREF (ids and pool rows past the split read nothing)
  auto refill = [&](int it, TileRawX& rw, bool& vr, int64_t& prr, int32_t& er) {
    const int64_t tn = r0 + (int64_t)(it + PREF) * kXTile;
    load_rows(resolve_row(tn + lrow, prr, vr), rw);
    prr = pool_row(tn + PREF * kXTile + lrow, er);
    er = fetch_id(tn + 2 * PREF * kXTile);
  };
  auto tile_step = [&](int it, TileRawX& raw, bool& v_raw, int64_t& prr, int32_t& er) {
    const int buf = it & 1;
    __bf16* yt = &ytile[buf][0];
    {
      // convert and store this thread's share of the tile (absent rows become zeros; a
      // wavefront whose rows all exist skips the masking)
      __bf16* dst = yt + lrow * kXRS;
      const uint64_t ball = ballot64(v_raw);
      auto put = [&](bool keep) {
#pragma unroll
        for (int i = 0; i < 7; i++) {
          const uint32_t w0 = keep ? raw.e[i][0] : 0u, w1 = keep ? raw.e[i][1] : 0u;
          const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
          const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
          const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
          const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
          *(bf16x8*)(dst + 64 * i + 8 * lk) =
              bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
        u32x4 v = raw.r;
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = keep ? v[e] : 0u;
        *(u32x4*)(dst + 448 + 8 * lk) = v;
      };
      if (ball == ~0ull) put(true);
      else put(v_raw);
      if (lane == 0) {
        uint32_t m8 = 0;
#pragma unroll
        for (int r = 0; r < 8; r++) m8 |= (uint32_t)((ball >> (8 * r)) & 1u) << r;
        s_mask[buf][hgl] = m8;
      }
    }
    if constexpr (PREF > 1) refill(it, raw, v_raw, prr, er);  // the slot's registers are free
    __syncthreads();
    const uint32_t mask = s_mask[buf][0] | (s_mask[buf][1] << 8) | (s_mask[buf][2] << 16) |
                          (s_mask[buf][3] << 24);
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
    if (mask != 0u) {
      // S^T for rows tb..tb+15 (S0) and tb+16..tb+31 (S1), even and odd chunks in separate
      // accumulators: four independent chains issue back to back (a dependent product waits
      // for its predecessor's result)
      // (two chains with two workgroups per CU, which cover each other's waits and have no
      // registers to spare)
      if constexpr (MINW == 1) {
        f32x4 S0e = S0, S0o = S0, S1e = S0, S1o = S0;
#pragma unroll
        for (int c = 0; c < NCH; c += 2) {
          const bf16x8 a0 = *(const bf16x8*)(yt + n * kXRS + 32 * c + 8 * g);
          const bf16x8 a1 = *(const bf16x8*)(yt + (16 + n) * kXRS + 32 * c + 8 * g);
          const bf16x8 b0 = *(const bf16x8*)(yt + n * kXRS + 32 * (c + 1) + 8 * g);
          const bf16x8 b1 = *(const bf16x8*)(yt + (16 + n) * kXRS + 32 * (c + 1) + 8 * g);
          S0e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[c], S0e, 0, 0, 0);
          S1e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[c], S1e, 0, 0, 0);
          S0o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, qf[c + 1], S0o, 0, 0, 0);
          S1o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, qf[c + 1], S1o, 0, 0, 0);
        }
        S0 = S0e + S0o;
        S1 = S1e + S1o;
      } else {
#pragma unroll
        for (int c = 0; c < NCH; c++) {
          const bf16x8 a0 = *(const bf16x8*)(yt + n * kXRS + 32 * c + 8 * g);
          const bf16x8 a1 = *(const bf16x8*)(yt + (16 + n) * kXRS + 32 * c + 8 * g);
          S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[c], S0, 0, 0, 0);
          S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[c], S1, 0, 0, 0);
        }
      }
      // Scheduling groups: the reads of QA chunks are in flight ahead of the products that use
      // them, so the LDS latency hides behind QA chunks of matrix work (left alone, the compiler
      // waits for each chunk's reads right before its products).
      constexpr int QA = MINW == 1 ? 4 : 1;  // two workgroups per CU cover each other instead
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * QA, 0);  // LDS reads
#pragma unroll
      for (int c = QA; c < NCH; c++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * QA, 0);
    }
    // one tile ahead: the next tile's loads go out now, after the products that needed the
    // registers of the row fragments
    if constexpr (PREF == 1) refill(it, raw, v_raw, prr, er);
    auto ytr = [&](int t) -> bf16x8 {
      const __bf16* base0 = yt + tr_row * kXRS + 16 * t + tr_col;
      const short4_t y0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)base0);
      const short4_t y1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(base0 + 16 * kXRS));
      return __builtin_bit_cast(bf16x8,
                                short8_t{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]});
    };
    if (mask != 0u) {
      // Y^T fragments of the PV products, read from LDS into a ring of PA pairs of 16-dim
      // tiles: the first PA pairs go out before the softmax, which hides their latency, and each
      // later pair PA pairs ahead of its products.
      constexpr int PA = MINW == 1 ? 4 : 1;
      constexpr int RF = 2 * PA;              // fragments in the ring
      constexpr int GRP = MINW == 1 ? 4 : 2;  // fragments per group of products
      bf16x8 yf[RF];
#pragma unroll
      for (int t = 0; t < RF; t++) yf[t] = ytr(t);
      // online softmax (base 2); lane holds rows 4g+i (S0) and 16+4g+i (S1) of head n. With every
      // row of the tile present (all but the edge tiles) the exponent is one fma of the raw score.
      const bool full = mask == 0xFFFFFFFFu;
      const float sc = p.scale_log2;
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[i] = S0[i];
        v[4 + i] = S1[i];
      }
      float tmax;
      if (full) {
        float hi = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        hi = fmaxf(hi, fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
        if (sc < 0.0f) {
          hi = fminf(fminf(v[0], v[1]), fminf(v[2], v[3]));
          hi = fminf(hi, fminf(fminf(v[4], v[5]), fminf(v[6], v[7])));
        }
        tmax = hi * sc;
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          v[i] = ((mask >> (4 * g + i)) & 1u) ? S0[i] * sc : -INFINITY;
          v[4 + i] = ((mask >> (16 + 4 * g + i)) & 1u) ? S1[i] * sc : -INFINITY;
        }
        tmax = v[0];
#pragma unroll
        for (int i = 1; i < 8; i++) tmax = fmaxf(tmax, v[i]);
      }
      tmax = max_row_groups(tmax);
      // lazy rescale: the reference max moves only when a head's max grows by more than 2^8
      const float m_new = fmaxf(m_run, tmax);
      if (__ballot(m_new > m_run + 8.0f)) {
        const float alpha = exp2f(m_run - m_new);  // 0 while nothing was accumulated
        if (__ballot(m_run != -INFINITY && alpha != 1.0f)) {
#pragma unroll
          for (int t = 0; t < NT; t++) O[t] *= alpha;
        }
        l_run *= alpha;
        m_run = m_new;
      }
      float P[8], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        // exponent <= 8; an absent row's -inf gives 0
        P[i] = __builtin_amdgcn_exp2f(full ? __builtin_fmaf(v[i], sc, -m_run) : v[i] - m_run);
        psum += P[i];
      }
      // The lo term of P carries bits 9-16 of each weight. With SKIPLO a wavefront leaves it out
      // of a tile when none of the tile's weights exceeds 1/16 of the weight its lane has already
      // summed for the same head (that partial sum is at most the head's final normaliser):
      // rows that small cannot dominate the output, and their rounding errors, of random sign and
      // at most 2^-8 of each weight, add up to well under the 1e-3 tolerance. A softmax with a
      // few dominant rows keeps the lo term on the tiles that hold them.
      bool lo = true;
      if constexpr (SKIPLO) {
        float pmax = fmaxf(fmaxf(fmaxf(P[0], P[1]), fmaxf(P[2], P[3])),
                           fmaxf(fmaxf(P[4], P[5]), fmaxf(P[6], P[7])));
        lo = __ballot(pmax > kLoSkipFrac * l_run) != 0ull;
      }
      l_run += psum;
      if constexpr (!SKIPLO) {
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          ph[e] = (__bf16)P[e];
          pl[e] = (__bf16)(P[e] - (float)ph[e]);
        }
        // a group's hi products, then its lo products: GRP independent chains
#pragma unroll
        for (int t = 0; t < NT; t += GRP) {
          bf16x8 y[GRP];
#pragma unroll
          for (int j = 0; j < GRP; j++) y[j] = yf[(t + j) % RF];
#pragma unroll
          for (int j = 0; j < GRP; j++)
            O[t + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y[j], ph, O[t + j], 0, 0, 0);
#pragma unroll
          for (int j = 0; j < GRP; j++)
            O[t + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y[j], pl, O[t + j], 0, 0, 0);
          if (t + RF < NT) {
#pragma unroll
            for (int j = 0; j < GRP; j++) yf[(t + j) % RF] = ytr(t + j + RF);
          }
        }
        // each group's products, then the reads of the group RF fragments ahead (2 transposing
        // reads per 16-dim tile)
#pragma unroll
        for (int t = 0; t < NT - RF; t += GRP) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * GRP, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * GRP, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * RF, 1);
      } else {
        // the hi products over all dims, then (when kept) the lo products in a second pass that
        // reads the Y^T fragments again: the pass is a block of its own after the first, so a
        // tile without it runs exactly the hi pass, and neither pass holds the other's registers
        auto pass = [&](const bf16x8& pw) {
#pragma unroll
          for (int t = 0; t < NT; t += GRP) {
            bf16x8 y[GRP];
#pragma unroll
            for (int j = 0; j < GRP; j++) y[j] = yf[(t + j) % RF];
#pragma unroll
            for (int j = 0; j < GRP; j++)
              O[t + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y[j], pw, O[t + j], 0, 0, 0);
            if (t + RF < NT) {
#pragma unroll
              for (int j = 0; j < GRP; j++) yf[(t + j) % RF] = ytr(t + j + RF);
            }
          }
#pragma unroll
          for (int t = 0; t < NT - RF; t += GRP) {
            __builtin_amdgcn_sched_group_barrier(0x008, GRP, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * GRP, 1);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, RF, 1);
        };
        bf16x8 ph;
#pragma unroll
        for (int e = 0; e < 8; e++) ph[e] = (__bf16)P[e];
        pass(ph);
        if (lo) {
          bf16x8 pl;
#pragma unroll
          for (int e = 0; e < 8; e++) pl[e] = (__bf16)(P[e] - (float)ph[e]);
#pragma unroll
          for (int t = 0; t < RF; t++) yf[t] = ytr(t);
          pass(pl);
        }
      }
    }
  };
  // The ring slots are compile-time indices: the loop is unrolled by the ring depth and runs
  // whole rounds of PREF tiles, where every step has the same loads in flight before it and so
  // waits for its own rows only (a step skipped inside the loop would make every wait drain all
  // loads). The last iters mod PREF tiles follow the loop.
  int it0 = 0;
  for (; it0 + PREF <= iters; it0 += PREF) {
#pragma unroll
    for (int k = 0; k < PREF; k++) tile_step(it0 + k, raw[k], v_raw[k], pr[k], ee[k]);
  }
#pragma unroll
  for (int k = 0; k < PREF - 1; k++)
    if (it0 + k < iters) tile_step(it0 + k, raw[k], v_raw[k], pr[k], ee[k]);

  // ---- write the output or this split's partial ----
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (head < p.H) {
    const float M = m_run, L = l_run;
    if (p.splits == 1) {
      float Mf = M, den = L, a = 1.0f;
      if (p.sink) {
        const float sg = p.sink[head] * kLog2e;
        Mf = fmaxf(M, sg);
        a = M == -INFINITY ? 0.0f : exp2f(M - Mf);
        den = L * a + exp2f(sg - Mf);
      }
      const float so = den > 0.0f ? a / den : 0.0f;
      float* op = p.out + ((int64_t)slot * p.H + head) * D + 4 * g;
#pragma unroll
      for (int t = 0; t < NT; t++) *(f32x4*)(op + 16 * t) = O[t] * so;
      if (p.lse && g == 0)
        p.lse[(int64_t)slot * p.H + head] = den > 0.0f ? (Mf + log2f(den)) * kLn2 : -INFINITY;
    } else {
      // partial row: acc[D], max, sum, 2 pad floats (16-byte aligned rows)
      float* pp = p.part + (((int64_t)slot * p.splits + split) * p.H + head) * (D + 4);
#pragma unroll
      for (int t = 0; t < NT; t++) *(f32x4*)(pp + 16 * t + 4 * g) = O[t];
      if (g == 0) {
        pp[D] = M;
        pp[D + 1] = L;
      }
    }
  }
}

// Combine the split partials of one (query, head) with the sink. Each thread owns D/128
// consecutive dims. The rows of up to 16 splits are loaded at once, before their weights are
// known (only the split maxima and sums wait for the weight computation), so one batch costs
// one memory round trip; absent splits read split 0 again and get weight 0, which keeps every
// load out of a branch.
constexpr int kMaxSplits = 64;
constexpr int kMergeBatch = 16;

template <int D>
__global__ __launch_bounds__(128) void attend_merge_kernel(const float* __restrict__ part,
                                                           int splits, int H,
                                                           const float* __restrict__ sink,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  constexpr int DPT = D / 128;
  typedef float vecD __attribute__((ext_vector_type(DPT)));
  const int hh = blockIdx.x, slot = blockIdx.y, t = threadIdx.x;
  const float* base = part + ((int64_t)slot * splits * H + hh) * (D + 4);
  const int64_t sstride = (int64_t)H * (D + 4);
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_den, s_mf;
  float ml = -INFINITY, ll = 0.0f;
  const float* mlp = base + (t < splits ? t : 0) * sstride + D;
  ml = mlp[0];
  ll = mlp[1];
  // the first batch of rows, in flight while the weights are computed
  vecD v[kMergeBatch];
#pragma unroll
  for (int j = 0; j < kMergeBatch; j++)
    v[j] = *(const vecD*)(base + (j < splits ? j : 0) * sstride + t * DPT);
  if (t >= splits) ml = -INFINITY, ll = 0.0f;
  // max over splits (and the sink) within the first wave
  if (t < 64) {
    float M = ml;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float Mf = M;
    const float sg = sink ? sink[hh] * kLog2e : 0.0f;
    if (sink) Mf = fmaxf(M, sg);
    const float wgt = (t < splits && ml != -INFINITY) ? exp2f(ml - Mf) : 0.0f;
    s_w[t] = wgt;
    float den = ll * wgt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
    if (t == 0) {
      s_den = den + (sink ? exp2f(sg - Mf) : 0.0f);
      s_mf = Mf;
    }
  }
  __syncthreads();
  const float den = s_den;
  vecD acc = {};
  for (int s0 = 0; s0 < splits; s0 += kMergeBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < kMergeBatch; j++) {
        const int sj = s0 + j < splits ? s0 + j : 0;
        v[j] = *(const vecD*)(base + sj * sstride + t * DPT);
      }
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; j++) {
      const float wgt = s0 + j < splits ? s_w[s0 + j] : 0.0f;
      acc += v[j] * wgt;
    }
  }
  const int64_t oo = (int64_t)slot * H + hh;
  vecD r;
#pragma unroll
  for (int e = 0; e < DPT; e++) r[e] = den > 0.0f ? acc[e] / den : 0.0f;
  *(vecD*)(out + oo * D + t * DPT) = r;
  if (t == 0 && lse) lse[oo] = den > 0.0f ? (s_mf + log2f(den)) * kLn2 : -INFINITY;
}

// Row splits: enough (query, split, head group) workgroups to fill the chip, at least `min_tiles`
// tiles per split, at most kMaxSplits splits.
static AttendPlan make_plan(int64_t base, int64_t tiles, int64_t want_wgs, int64_t min_tiles) {
  AttendPlan pl;
  int64_t want = (want_wgs + base - 1) / base;
  int64_t cap = (tiles + min_tiles - 1) / min_tiles;
  if (cap < 1) cap = 1;
  int64_t S = want < cap ? want : cap;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  const int64_t tps = tiles > 0 ? (tiles + S - 1) / S : 1;
  pl.splits = tiles > 0 ? (int)((tiles + tps - 1) / tps) : 1;
  pl.rows_per_split = (int)(tps * kTile);
  return pl;
}

// attend_kernel: workgroups of 4 wavefronts over one head group of 16, each wavefront its own tiles.
AttendPlan attend_plan(int B, int Q, int H, int D, int64_t max_rows) {
  (void)D;
  const int hg = (H + 15) / 16;
  AttendPlan pl = make_plan((int64_t)B * Q * hg, (max_rows + kTile - 1) / kTile, 512, kWaves);
  pl.head_groups = hg;
  return pl;
}

// attend_x_kernel: workgroups of 4 wavefronts over one (query, row split, block of 64 heads). Grids
// of up to 256 workgroups take the one-per-CU build, larger ones the two-per-CU build.
static AttendPlan attend_x_plan(int B, int Q, int H, int64_t max_rows) {
  const int hb = (H + 63) / 64;
  const int64_t base = (int64_t)B * Q * hb;
  // Each split writes a 64-head partial (128 KB, as large as 228 rows of input), yet a 32-row
  // tile costs about 1.7 us of matrix and vector issue, so parallelism wins over partial bytes:
  // measured at 16 sequences, splits of 3 tiles (12 per sequence) beat 4 tiles by 9% and 6 tiles
  // by 25%; at 4 sequences, 2 tiles beat 1, 3 and 4.
  const int min_tiles = base >= 16 ? 3 : 2;
  const int64_t tiles = (max_rows + kXTile - 1) / kXTile;
  // Up to 240 workgroups, one per CU: a workgroup takes a CU's whole register file, and the
  // 16 CUs left over (two per XCD) keep room for a kernel running concurrently on another stream.
  // In a decode step the CSA layer's top-k (16 workgroups of 1,024 threads) otherwise waits for
  // the whole HCA attention to finish. Dense attention over long row sets (64 tiles or more per
  // query) for 20 or more (query, head block) units targets 480 workgroups instead, of the
  // two-per-CU build: measured at 8,320 rows, 20 to 64 sequences ran 1.5-10% faster, and the
  // 4 x 5-query decode step 142.5 against 151.3 us (its two attention grids then share CUs).
  // Sparse attention (36 tiles) at 32 and 64 sequences ran 15-20% slower that way, and the
  // 16-sequence step 139 against 133 us, so both keep 240.
  const int64_t want = base >= 20 && tiles >= 64 ? 480 : 240;
  AttendPlan pl = make_plan(base, tiles, want, min_tiles);
  pl.head_groups = hb;
  return pl;
}

static size_t partial_bytes(int B, int Q, int H, int D, const AttendPlan& pl) {
  return pl.splits <= 1 ? 0 : (size_t)B * Q * pl.splits * H * (D + 4) * sizeof(float);
}

size_t attend_workspace_bytes(int B, int Q, int H, int D, int64_t max_rows) {
  // D = 512 rows are E4M3 + bf16: bf16 queries take attend_x_kernel, fp32 queries attend_kernel
  size_t need = partial_bytes(B, Q, H, D, attend_plan(B, Q, H, D, max_rows));
  if (D == 512) {
    const size_t x = partial_bytes(B, Q, H, D, attend_x_plan(B, Q, H, max_rows));
    need = x > need ? x : need;
  }
  return need;
}

template <int FMT, int QDT>
static hipError_t launch_fmt(const AttendArgs& a, const AttendK& k, dim3 grid, hipStream_t s) {
  if (a.idx) a.prof.launch(attend_kernel<FMT, QDT, false>, grid, dim3(256), s, k);
  else a.prof.launch(attend_kernel<FMT, QDT, true>, grid, dim3(256), s, k);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a) {
  hipStream_t s = (hipStream_t)a.stream;
  const bool shared_tiles = a.fmt == CSAH_FMT_ROW_E4M3_BF16 && a.q_dtype == CSAH_DT_BF16;
  const AttendPlan pl = shared_tiles ? attend_x_plan(a.B, a.Q, a.H, a.max_rows)
                                     : attend_plan(a.B, a.Q, a.H, a.D, a.max_rows);
  AttendK k;
  k.q = a.q;
  k.H = a.H;
  k.cache = (const uint8_t*)a.cache;
  k.cmap = a.cmap;
  k.N = a.N;
  k.idx = a.idx;
  k.k = a.k;
  k.m = a.m;
  k.win = (const uint8_t*)a.win;
  k.wstride = a.win_seq_stride;
  k.w = a.w;
  k.pos = a.pos;
  k.sink = a.sink;
  k.scale_log2 = a.scale * kLog2e;
  k.Q = a.Q;
  k.splits = pl.splits;
  k.rows_per_split = pl.rows_per_split;
  k.hg = pl.head_groups;
  k.slots = a.B * a.Q;
  k.out = a.out;
  k.lse = a.lse;
  k.part = (float*)a.ws;
  // 1-D grid padded to whole XCD rounds (8 x head groups); padding workgroups exit at once
  const int64_t units = (int64_t)pl.splits * a.B * a.Q;
  const int64_t per_round = 8LL * pl.head_groups;
  dim3 grid((unsigned)(((units + 7) / 8) * per_round));
  hipError_t e;
  if (shared_tiles) {
    const dim3 blk(256);
    const bool paged = a.cmap.table != nullptr, dense = a.idx == nullptr;
    if (grid.x <= 256) {
      if (paged) {
        if (dense) a.prof.launch(attend_x_kernel<true, true, 1, false>, grid, blk, s, k);
        else a.prof.launch(attend_x_kernel<false, true, 1, false>, grid, blk, s, k);
      } else {
        if (dense) a.prof.launch(attend_x_kernel<true, false, 1, false>, grid, blk, s, k);
        else a.prof.launch(attend_x_kernel<false, false, 1, false>, grid, blk, s, k);
      }
    } else if (pl.rows_per_split >= 64 * kXTile) {
      if (paged) {
        if (dense) a.prof.launch(attend_x_kernel<true, true, 2, true>, grid, blk, s, k);
        else a.prof.launch(attend_x_kernel<false, true, 2, true>, grid, blk, s, k);
      } else {
        if (dense) a.prof.launch(attend_x_kernel<true, false, 2, true>, grid, blk, s, k);
        else a.prof.launch(attend_x_kernel<false, false, 2, true>, grid, blk, s, k);
      }
    } else {
      if (paged) {
        if (dense) a.prof.launch(attend_x_kernel<true, true, 2, false>, grid, blk, s, k);
        else a.prof.launch(attend_x_kernel<false, true, 2, false>, grid, blk, s, k);
      } else {
        if (dense) a.prof.launch(attend_x_kernel<true, false, 2, false>, grid, blk, s, k);
        else a.prof.launch(attend_x_kernel<false, false, 2, false>, grid, blk, s, k);
      }
    }
    e = hipGetLastError();
  } else if (a.fmt == CSAH_FMT_ROW_E4M3_BF16)
    e = launch_fmt<CSAH_FMT_ROW_E4M3_BF16, CSAH_DT_F32>(a, k, grid, s);
  else
    e = a.q_dtype == CSAH_DT_BF16 ? launch_fmt<CSAH_FMT_ROW_F32, CSAH_DT_BF16>(a, k, grid, s)
                                  : launch_fmt<CSAH_FMT_ROW_F32, CSAH_DT_F32>(a, k, grid, s);
  if (e != hipSuccess || pl.splits == 1) return e;
  dim3 mg((unsigned)a.H, (unsigned)(a.B * a.Q));
  if (a.D == 512)
    attend_merge_kernel<512><<<mg, 128, 0, s>>>(k.part, pl.splits, a.H, a.sink, a.out, a.lse);
  else
    attend_merge_kernel<128><<<mg, 128, 0, s>>>(k.part, pl.splits, a.H, a.sink, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace csah
