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
//   - The QK A-operand is loaded straight from HBM (lane l: row l%16, 8 dims at 8*(l/16)), converted
//     in registers, and the same registers are written transposed into a per-wavefront LDS tile
//     Yt[d][slot] that feeds the PV A-operand with 16-byte reads. Slot order matches the C layout of
//     S^T, so P never moves between lanes. The 16-byte segments of a Yt row are XOR-swizzled by
//     (d / 8) % 4 to spread the transposing writes over the LDS banks.
//   - Online softmax in base 2 (running max per head, lazy rescale of the accumulators only when
//     the max moves).
// Grid: (row splits x head groups of 16, sequences x queries). The 4 wavefronts of a workgroup take
// 32-row tiles of the split in turn and are merged in LDS at the end; with one split the workgroup
// applies the sink and writes the output, otherwise it writes (max, sum, acc) partials that
// attend_merge_kernel combines with the sink.
#include "csah_internal.h"
#include "device_common.h"

namespace csah {

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
  int64_t cstride, N;
  const int32_t* idx;
  int k, m;
  const uint8_t* win;
  int64_t wstride;
  int w;
  const int64_t* pos;
  const float* sink;
  float scale_log2;
  int Q, splits, rows_per_split, hg;
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

// 8 consecutive dims [32c + 8g, +8) of one row as bf16 (hi, and lo for fp32 rows).
template <int FMT>
__device__ __forceinline__ void load_row_frag(const uint8_t* row, bool valid, int c, int g,
                                              bf16x8& hi, bf16x8& lo) {
  if constexpr (FMT == CSAH_FMT_ROW_E4M3_BF16) {
    if (!valid) {
      hi = bf16x8{};
      return;
    }
    if (c < 14) {
      const u32x2 v = *(const u32x2*)(row + 32 * c + 8 * g);
      bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
      bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
      bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
      bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
      hi = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    } else {
      const u32x4 v = *(const u32x4*)(row + 448 + 64 * (c - 14) + 16 * g);
      hi = __builtin_bit_cast(bf16x8, v);
    }
  } else {
    if (!valid) {
      hi = bf16x8{};
      lo = bf16x8{};
      return;
    }
    const f32x4 a = *(const f32x4*)(row + 4 * (32 * c + 8 * g));
    const f32x4 b = *(const f32x4*)(row + 4 * (32 * c + 8 * g) + 16);
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    float r[8];
    hi = pack_bf16x8(x);
#pragma unroll
    for (int e = 0; e < 8; e++) r[e] = x[e] - (float)hi[e];
    lo = pack_bf16x8(r);
  }
}

// LDS element index of Yt[d][slot] inside one wavefront's tile (32 slots per row, swizzled).
__device__ __forceinline__ int yt_index(int d, int slot) {
  const int seg = (slot >> 3) ^ ((d >> 3) & 3);
  return d * kTile + seg * 8 + (slot & 7);
}

template <int FMT, int QDT, bool DENSE>
__global__ __launch_bounds__(256, 1) void attend_kernel(AttendK p) {
  using C = RowCfg<FMT>;
  constexpr int D = C::D, NCH = C::NCH, YS = C::YS, NT = D / 16;
  constexpr int QS = QDT == CSAH_DT_F32 ? 2 : 1;
  constexpr int YT_ELEMS = D * kTile;  // bf16 elements per wavefront per split term
  constexpr int LDS_YT = kWaves * YS * YT_ELEMS * 2;
  constexpr int LDS_COMB = kWaves * 16 * D * 4;
  constexpr int LDS_BYTES = LDS_YT > LDS_COMB ? LDS_YT : LDS_COMB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  __shared__ float s_ml[kWaves][16][2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int slot = blockIdx.y;
  const int b = slot / p.Q, qi = slot - b * p.Q;
  const int split = blockIdx.x / p.hg, hgi = blockIdx.x - split * p.hg;
  const int head = hgi * 16 + n;
  const bool head_ok = head < p.H;

  // ---- query fragments: B operand of S^T = Y Q^T (k = dims 32c + 8g + e, n = head) ----
  bf16x8 qf[QS][NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    if (!head_ok) {
#pragma unroll
      for (int s = 0; s < QS; s++) qf[s][c] = bf16x8{};
      continue;
    }
    const int64_t qo = ((int64_t)slot * p.H + head) * D + 32 * c + 8 * g;
    if constexpr (QDT == CSAH_DT_BF16) {
      qf[0][c] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const uint16_t*)p.q + qo));
    } else {
      const float* qp = (const float*)p.q + qo;
      const f32x4 a = *(const f32x4*)qp, bb = *(const f32x4*)(qp + 4);
      float x[8] = {a[0], a[1], a[2], a[3], bb[0], bb[1], bb[2], bb[3]}, r[8];
      qf[0][c] = pack_bf16x8(x);
#pragma unroll
      for (int e = 0; e < 8; e++) r[e] = x[e] - (float)qf[0][c][e];
      qf[QS - 1][c] = pack_bf16x8(r);
    }
  }

  // ---- the logical row range of this split ----
  const int64_t pos_b = p.pos[b];
  int64_t Rc;
  if constexpr (DENSE) {
    int64_t nv = (pos_b + qi + 1) / p.m;
    Rc = nv < 0 ? 0 : (nv > p.N ? p.N : nv);
  } else {
    Rc = p.k;
  }
  const int64_t R = Rc + p.w;
  const int64_t r0 = (int64_t)split * p.rows_per_split;
  const int64_t r1 = r0 + p.rows_per_split < R ? r0 + p.rows_per_split : R;

  auto row_ptr = [&](int64_t j, bool& valid) -> const uint8_t* {
    valid = false;
    if (j >= r1) return nullptr;
    if (j < Rc) {
      int64_t e;
      if constexpr (DENSE) {
        e = j;
      } else {
        e = p.idx[(int64_t)slot * p.k + j];
        if (e < 0 || e >= p.N) return nullptr;
      }
      valid = true;
      return p.cache + ((int64_t)b * p.cstride + e) * C::RB;
    }
    const int64_t r = qi + (j - Rc);                 // window buffer row
    const int64_t rpos = pos_b - (p.w - 1) + r;      // its token position
    if (rpos < 0) return nullptr;
    valid = true;
    return p.win + ((int64_t)b * p.wstride + r) * C::RB;
  };

  __bf16* yt = (__bf16*)smem + wave * YS * YT_ELEMS;
  f32x4 O[NT];
#pragma unroll
  for (int t = 0; t < NT; t++) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const int slot0 = 8 * (n >> 2) + (n & 3);  // Yt slot of tile row n; row 16+n uses slot0 + 4

  for (int64_t tb = r0 + (int64_t)kTile * wave; tb < r1; tb += (int64_t)kTile * kWaves) {
    bool vm;
    (void)row_ptr(tb + (lane & 31), vm);
    const uint32_t mask = (uint32_t)ballot64(vm);
    if (mask == 0u) continue;
    bool v0, v1;
    const uint8_t* p0 = row_ptr(tb + n, v0);
    const uint8_t* p1 = row_ptr(tb + 16 + n, v1);

    // S^T for rows tb..tb+15 (S0) and tb+16..tb+31 (S1); stage Y^T in LDS on the way
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      bf16x8 a0h, a0l, a1h, a1l;
      load_row_frag<FMT>(p0, v0, c, g, a0h, a0l);
      load_row_frag<FMT>(p1, v1, c, g, a1h, a1l);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0h, qf[0][c], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1h, qf[0][c], S1, 0, 0, 0);
      if constexpr (QS == 2) {
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0h, qf[1][c], S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1h, qf[1][c], S1, 0, 0, 0);
      }
      if constexpr (YS == 2) {
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0l, qf[0][c], S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1l, qf[0][c], S1, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int d = 32 * c + 8 * g + e;
        yt[yt_index(d, slot0)] = a0h[e];
        yt[yt_index(d, slot0 + 4)] = a1h[e];
        if constexpr (YS == 2) {
          yt[YT_ELEMS + yt_index(d, slot0)] = a0l[e];
          yt[YT_ELEMS + yt_index(d, slot0 + 4)] = a1l[e];
        }
      }
    }

    // online softmax (base 2); lane holds rows 4g+i (S0) and 16+4g+i (S1) of head n
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[i] = ((mask >> (4 * g + i)) & 1u) ? S0[i] * p.scale_log2 : -INFINITY;
      v[4 + i] = ((mask >> (16 + 4 * g + i)) & 1u) ? S1[i] * p.scale_log2 : -INFINITY;
    }
    float tmax = v[0];
#pragma unroll
    for (int i = 1; i < 8; i++) tmax = fmaxf(tmax, v[i]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float P[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      P[i] = exp2f(v[i] - m_new);
      psum += P[i];
    }
    l_run = fmaf(l_run, alpha, psum);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < NT; t++) O[t] *= alpha;
    }
    m_run = m_new;
    bf16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      ph[e] = (__bf16)P[e];
      pl[e] = (__bf16)(P[e] - (float)ph[e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += Y^T P^T
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int d = 16 * t + n;
      const bf16x8 ya = *(const bf16x8*)(yt + yt_index(d, 8 * g));
      O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ya, ph, O[t], 0, 0, 0);
      O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ya, pl, O[t], 0, 0, 0);
      if constexpr (YS == 2) {
        const bf16x8 yl = *(const bf16x8*)(yt + YT_ELEMS + yt_index(d, 8 * g));
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yl, ph, O[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the 4 wavefronts ----
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  __syncthreads();
  float* comb = (float*)smem;  // [wave][16 heads][D]
#pragma unroll
  for (int t = 0; t < NT; t++)
#pragma unroll
    for (int i = 0; i < 4; i++) comb[(wave * 16 + n) * D + 16 * t + 4 * g + i] = O[t][i];
  if (g == 0) {
    s_ml[wave][n][0] = m_run;
    s_ml[wave][n][1] = l_run;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += 256) {
    const int hl = e / D, d = e - hl * D;
    const int hh = hgi * 16 + hl;
    if (hh >= p.H) continue;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; wv++) M = fmaxf(M, s_ml[wv][hl][0]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; wv++) {
      const float mw = s_ml[wv][hl][0];
      const float om = mw == -INFINITY ? 0.0f : exp2f(mw - M);
      L = fmaf(s_ml[wv][hl][1], om, L);
      acc = fmaf(comb[(wv * 16 + hl) * D + d], om, acc);
    }
    if (p.splits == 1) {
      float Mf = M, den = L;
      if (p.sink) {
        const float sg = p.sink[hh] * kLog2e;
        Mf = fmaxf(M, sg);
        const float a = M == -INFINITY ? 0.0f : exp2f(M - Mf);
        den = L * a + exp2f(sg - Mf);
        acc *= a;
      }
      const int64_t oo = ((int64_t)slot * p.H + hh);
      p.out[oo * D + d] = den > 0.0f ? acc / den : 0.0f;
      if (d == 0 && p.lse) p.lse[oo] = den > 0.0f ? (Mf + log2f(den)) * kLn2 : -INFINITY;
    } else {
      float* pp = p.part + (((int64_t)slot * p.splits + split) * p.H + hh) * (D + 2);
      pp[2 + d] = acc;
      if (d == 0) {
        pp[0] = M;
        pp[1] = L;
      }
    }
  }
}

// Combine the split partials of one (query, head) with the sink.
template <int D>
__global__ __launch_bounds__(128) void attend_merge_kernel(const float* __restrict__ part,
                                                           int splits, int H,
                                                           const float* __restrict__ sink,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int hh = blockIdx.x, slot = blockIdx.y;
  const float* base = part + ((int64_t)slot * splits * H + hh) * (D + 2);
  const int64_t sstride = (int64_t)H * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < splits; s++) M = fmaxf(M, base[s * sstride]);
  float Mf = M;
  float sg = 0.0f;
  if (sink) {
    sg = sink[hh] * kLog2e;
    Mf = fmaxf(M, sg);
  }
  float den = sink ? exp2f(sg - Mf) : 0.0f;
  for (int s = 0; s < splits; s++) {
    const float ms = base[s * sstride];
    if (ms != -INFINITY) den = fmaf(base[s * sstride + 1], exp2f(ms - Mf), den);
  }
  const int64_t oo = (int64_t)slot * H + hh;
  for (int d = threadIdx.x; d < D; d += 128) {
    float acc = 0.0f;
    for (int s = 0; s < splits; s++) {
      const float ms = base[s * sstride];
      if (ms != -INFINITY) acc = fmaf(base[s * sstride + 2 + d], exp2f(ms - Mf), acc);
    }
    out[oo * D + d] = den > 0.0f ? acc / den : 0.0f;
  }
  if (threadIdx.x == 0 && lse) lse[oo] = den > 0.0f ? (Mf + log2f(den)) * kLn2 : -INFINITY;
}

AttendPlan attend_plan(int B, int Q, int H, int D, int64_t max_rows) {
  (void)D;
  AttendPlan pl;
  pl.head_groups = (H + 15) / 16;
  const int64_t tiles = (max_rows + kTile - 1) / kTile;
  const int64_t base = (int64_t)B * Q * pl.head_groups;
  int64_t want = (512 + base - 1) / base;
  int64_t cap = (tiles + kWaves - 1) / kWaves;
  if (cap < 1) cap = 1;
  int64_t S = want < cap ? want : cap;
  if (S < 1) S = 1;
  int64_t tps = tiles > 0 ? (tiles + S - 1) / S : 1;
  S = tiles > 0 ? (tiles + tps - 1) / tps : 1;
  pl.splits = (int)S;
  pl.rows_per_split = (int)(tps * kTile);
  return pl;
}

size_t attend_workspace_bytes(int B, int Q, int H, int D, int64_t max_rows) {
  AttendPlan pl = attend_plan(B, Q, H, D, max_rows);
  if (pl.splits <= 1) return 0;
  return (size_t)B * Q * pl.splits * H * (D + 2) * sizeof(float);
}

template <int FMT, int QDT>
static hipError_t launch_fmt(const AttendArgs& a, const AttendK& k, dim3 grid, hipStream_t s) {
  if (a.idx) attend_kernel<FMT, QDT, false><<<grid, 256, 0, s>>>(k);
  else attend_kernel<FMT, QDT, true><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a) {
  hipStream_t s = (hipStream_t)a.stream;
  AttendPlan pl = attend_plan(a.B, a.Q, a.H, a.D, a.max_rows);
  AttendK k;
  k.q = a.q;
  k.H = a.H;
  k.cache = (const uint8_t*)a.cache;
  k.cstride = a.cache_seq_stride;
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
  k.out = a.out;
  k.lse = a.lse;
  k.part = (float*)a.ws;
  dim3 grid((unsigned)(pl.splits * pl.head_groups), (unsigned)(a.B * a.Q));
  hipError_t e;
  if (a.fmt == CSAH_FMT_ROW_E4M3_BF16)
    e = a.q_dtype == CSAH_DT_BF16 ? launch_fmt<CSAH_FMT_ROW_E4M3_BF16, CSAH_DT_BF16>(a, k, grid, s)
                                  : launch_fmt<CSAH_FMT_ROW_E4M3_BF16, CSAH_DT_F32>(a, k, grid, s);
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
