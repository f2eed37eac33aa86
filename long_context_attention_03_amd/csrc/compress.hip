// compress.hip -- kv_compress: softmax-gated pooling of m consecutive tokens into one entry.
//
// [EXPL] "DeepSeek V4 Architecture Explained: CSA, HCA, mHC and Muon", section "How
// compress-then-sparsify attention works": a group of m consecutive tokens' keys and values is
// folded into one entry using trainable compression weights, a softmax over the group and
// learnable positional biases. [LLMB] "Inside DeepSeek-V4 ...", sections "1. Compressed Sparse
// Attention (CSA)" (factor 4) and "2. Heavily Compressed Attention (HCA)" (factor 128).
//
//   z_t = w . x_t + beta[t - g m],  pi = softmax(z),  c_g = sum_t pi_t x_t.
//
// Lane l of a wavefront owns DPL = D/64 consecutive dimensions, so every token row is read with
// one coalesced vector load per lane. Tokens go in batches of 8 whose loads and gate reductions
// (symmetric wavefront exchanges) are in flight together. The softmax is evaluated online (running max,
// running denominator, running weighted sum), which keeps a group of any size in registers. Short
// spans (up to 16 tokens) take one wavefront each; longer ones take a workgroup of 4 (up to 64)
// or 8 wavefronts that pool a share of the tokens each and merge their states in LDS. The pooled
// row is encoded in the output format and written with vector stores. HBM traffic is one read of
// the raw rows and one write of the compressed rows. With RoPE (csah_kv_compress_rope) the pooled row's rotary pairs
// are turned in fp64 before encoding, at the position of the last token of the entry's group.
#include "csah_internal.h"
#include "device_common.h"

namespace csah {

template <int DPL, bool RAW_BF16>
__device__ __forceinline__ void load_token(const void* raw, int64_t row, int lane, float* x) {
  constexpr int D = DPL * 64;
  if constexpr (RAW_BF16) {
    const uint16_t* p = (const uint16_t*)raw + row * D + lane * DPL;
    if constexpr (DPL >= 8) {
#pragma unroll
      for (int v = 0; v < DPL / 8; v++) {
        u32x4 w = *(const u32x4*)(p + 8 * v);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          x[8 * v + 2 * e] = u2f(w[e] << 16);
          x[8 * v + 2 * e + 1] = u2f(w[e] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; e++) x[e] = u2f((uint32_t)p[e] << 16);
    }
  } else {
    const float* p = (const float*)raw + row * D + lane * DPL;
    if constexpr (DPL >= 4) {
#pragma unroll
      for (int v = 0; v < DPL / 4; v++) {
        f32x4 w = *(const f32x4*)(p + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; e++) x[4 * v + e] = w[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; e++) x[e] = p[e];
    }
  }
}

constexpr int kTokBatch = 8;  // tokens whose loads and gate reductions are in flight together

// Sum over the 64 lanes, in every lane, by symmetric exchanges only (quad swaps, half-row and
// row mirrors, gfx950's 16- and 32-lane swaps): both lanes of each pairing add the same two
// values, so every lane ends with the bit-identical sum, and no step goes through LDS.
__device__ __forceinline__ float wave_sum_all(float v) {
  v += u2f(__builtin_amdgcn_mov_dpp(f2u(v), 0xB1, 0xF, 0xF, true));   // lanes i ^ 1
  v += u2f(__builtin_amdgcn_mov_dpp(f2u(v), 0x4E, 0xF, 0xF, true));   // lanes i ^ 2
  v += u2f(__builtin_amdgcn_mov_dpp(f2u(v), 0x141, 0xF, 0xF, true));  // half-row mirror
  v += u2f(__builtin_amdgcn_mov_dpp(f2u(v), 0x140, 0xF, 0xF, true));  // row mirror
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v = u2f(a[0]) + u2f(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return u2f(c[0]) + u2f(c[1]);
}

// Entry g (after `skip` context-only groups) pools the `span` tokens that end with the last token
// of group g, [m(g+1) - span, m(g+1)); tokens before the start of the buffer are left out and the
// positional bias is indexed by the token's place in the span. span = m: one entry per group.
// WAVES = 1: one wavefront per entry, 4 entries per workgroup (short spans).
// WAVES = 4 or 8: one workgroup per entry; wavefront w pools a share of the span and the
//            online-softmax states (max, sum, weighted sum) are merged in LDS. With 8
//            wavefronts (spans past 64 tokens) a wavefront loads two batches before it pools
//            the first, so a 128-token group costs one memory round trip.
template <int DPL, bool RAW_BF16, int OUT_FMT, int WAVES, bool ROPE>
__global__ __launch_bounds__(64 * (WAVES == 1 ? 4 : WAVES)) void kv_compress_kernel(
    const void* __restrict__ raw, int64_t raw_seq_stride, int B, int64_t G, int m, int span,
    int64_t skip, const float* __restrict__ w, const float* __restrict__ beta,
    uint8_t* __restrict__ out_rows, EntryMap omap, int64_t first_entry,
    uint8_t* __restrict__ out_scales, const int64_t* __restrict__ tok_pos, int rope_dims,
    double rope_base) {
  constexpr int D = DPL * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gid = WAVES == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
  if (gid >= (int64_t)B * G) return;  // uniform per wavefront (WAVES = 1) or workgroup
  const int64_t b = gid / G, g = gid - b * G;  // g: output row; group g + skip

  float wv[DPL];
#pragma unroll
  for (int e = 0; e < DPL; e++) wv[e] = w[lane * DPL + e];

  // span positions [jmin, span) hold tokens (the ones before the buffer start are left out)
  const int64_t first = (int64_t)m * (g + skip + 1) - span;  // token at span position 0
  const int jmin = first < 0 ? (int)(-first) : 0;
  int t_begin = jmin, t_end = span;
  if constexpr (WAVES > 1) {
    const int per = (span - jmin + WAVES - 1) / WAVES;
    t_begin = jmin + wave * per;
    t_end = t_begin + per < span ? t_begin + per : span;
  }
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; e++) acc[e] = 0.0f;
  float M = -INFINITY, L = 0.0f;
  const int64_t row0 = b * raw_seq_stride + first;  // + j >= 0 for every position read
  // NB batches of tokens are loaded before the first is pooled (their loads in flight together)
  constexpr int NB = (WAVES >= 8 && DPL <= 8) ? 2 : 1;
  for (int t00 = t_begin; t00 < t_end; t00 += NB * kTokBatch) {
    float xb[NB][kTokBatch][DPL];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int u = 0; u < kTokBatch; u++) {
        const int tt = t00 + nb * kTokBatch + u;
        const int t = tt < t_end ? tt : t_end - 1;  // clamped: loads stay unconditional
        load_token<DPL, RAW_BF16>(raw, row0 + t, lane, xb[nb][u]);
      }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
    const int t0 = t00 + nb * kTokBatch;
    float (&x)[kTokBatch][DPL] = xb[nb];
    float z[kTokBatch];
#pragma unroll
    for (int u = 0; u < kTokBatch; u++) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; e++) s = fmaf(wv[e], x[u][e], s);
      z[u] = s;
    }
#pragma unroll
    for (int u = 0; u < kTokBatch; u++) z[u] = wave_sum_all(z[u]);
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTokBatch; u++) {
      z[u] = t0 + u < t_end ? z[u] + beta[t0 + u] : -INFINITY;
      bmax = fmaxf(bmax, z[u]);
    }
    const float Mn = fmaxf(M, bmax);
    // 0 on the first batch (M = -inf); a batch past the span end (Mn = M = -inf) changes nothing
    const float sc = Mn == -INFINITY ? 1.0f : expf(M - Mn);
#pragma unroll
    for (int e = 0; e < DPL; e++) acc[e] *= sc;
    L *= sc;
#pragma unroll
    for (int u = 0; u < kTokBatch; u++) {
      const float p = expf(z[u] - Mn);  // 0 for padding tokens
#pragma unroll
      for (int e = 0; e < DPL; e++) acc[e] = fmaf(p, x[u][e], acc[e]);
      L += p;
    }
    M = Mn;
    }
  }
  if constexpr (WAVES > 1) {
    __shared__ float s_acc[WAVES][D];
    __shared__ float s_ml[WAVES][2];
#pragma unroll
    for (int e = 0; e < DPL; e++) s_acc[wave][lane * DPL + e] = acc[e];
    if (lane == 0) {
      s_ml[wave][0] = M;
      s_ml[wave][1] = L;
    }
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < WAVES; v++) Mt = fmaxf(Mt, s_ml[v][0]);
    L = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; e++) acc[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; v++) {
      const float mv = s_ml[v][0];
      const float f = mv == -INFINITY ? 0.0f : expf(mv - Mt);
      L = fmaf(s_ml[v][1], f, L);
#pragma unroll
      for (int e = 0; e < DPL; e++) acc[e] = fmaf(s_acc[v][lane * DPL + e], f, acc[e]);
    }
  }
  float c[DPL];
#pragma unroll
  for (int e = 0; e < DPL; e++) c[e] = acc[e] / L;
  if constexpr (ROPE) {
    // RoPE before encoding: the rotary pairs (the last rope_dims dims) turn, in fp64, by the
    // position of the last token of the entry's group. Lane l computes the (cos, sin) of pair
    // jb + l of each round of 64 pairs, and the lanes holding a pair fetch them by shuffles, so a
    // wavefront waits for one sine and cosine per round instead of one per pair it holds.
    const double p = (double)(tok_pos[b] + (int64_t)m * (g + skip + 1) - 1);
    const int r0 = D - rope_dims;  // even, so a pair never straddles two lanes when DPL >= 2
    const int np = rope_dims / 2;
    float other = 0.0f;
    if constexpr (DPL == 1) other = __shfl_xor(c[0], 1, 64);  // the pair's other dim
    for (int jb = 0; jb < np; jb += 64) {  // uniform: every lane takes part in the shuffles
      double cl = 1.0, sl = 0.0;
      if (jb + lane < np) rope_cos_sin(p, jb + lane, rope_dims, rope_base, false, cl, sl);
      if constexpr (DPL == 1) {
        const int src = ((lane - r0) >> 1) - jb;
        const double cs = __shfl(cl, src & 63, 64), sn = __shfl(sl, src & 63, 64);
        if (lane >= r0 && src >= 0 && src < 64) {
          const bool odd = lane & 1;
          const double x0 = odd ? other : c[0], x1 = odd ? c[0] : other;
          c[0] = (float)(odd ? x0 * sn + x1 * cs : x0 * cs - x1 * sn);
        }
      } else {
#pragma unroll
        for (int e = 0; e < DPL; e += 2) {
          const int d = lane * DPL + e;
          const int src = ((d - r0) >> 1) - jb;
          const double cs = __shfl(cl, src & 63, 64), sn = __shfl(sl, src & 63, 64);
          if (d >= r0 && src >= 0 && src < 64) {
            const double x0 = c[e], x1 = c[e + 1];
            c[e] = (float)(x0 * cs - x1 * sn);
            c[e + 1] = (float)(x0 * sn + x1 * cs);
          }
        }
      }
    }
  }
  const int64_t orow = omap.row((int)b, first_entry + g);
  if constexpr (OUT_FMT == CSAH_FMT_ROW_F32) {
    float* o = (float*)out_rows + orow * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; e++) o[e] = c[e];
  } else if constexpr (OUT_FMT == CSAH_FMT_ROW_E4M3_BF16) {
    // D = 512: lanes 0..55 hold dims 0..447 (E4M3), lanes 56..63 dims 448..511 (bf16).
    static_assert(DPL == 8, "E4M3+bf16 rows are 512 wide");
    uint8_t* o = out_rows + orow * (int64_t)(D + 64);
    if (lane < 56) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; e++) lo |= f32_to_e4m3(c[e]) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; e++) hi |= f32_to_e4m3(c[4 + e]) << (8 * e);
      *(u32x2*)(o + 8 * lane) = u32x2{lo, hi};
    } else {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        bf16x2 p2 = {(__bf16)c[2 * e], (__bf16)c[2 * e + 1]};
        v[e] = __builtin_bit_cast(uint32_t, p2);
      }
      *(u32x4*)(o + 448 + 16 * (lane - 56)) = v;
    }
  } else {
    // MX block of 32 dims = 32/DPL lanes; shared exponent floor(log2 amax) - 2.
    constexpr int LPB = 32 / DPL;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; e++) amax = fmaxf(amax, fabsf(c[e]));
#pragma unroll
    for (int o = 1; o < LPB; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int sexp;
    if (amax == 0.0f) sexp = 0;
    else {
      int ef = (int)((f2u(amax) >> 23) & 255u);  // biased exponent (0 for subnormals)
      sexp = ef - 127 - 2;
      sexp = sexp < -127 ? -127 : (sexp > 127 ? 127 : sexp);
    }
    uint8_t* o = out_rows + orow * (int64_t)(D / 2) + lane * (DPL / 2);
    uint32_t nib[DPL];
#pragma unroll
    for (int e = 0; e < DPL; e++) nib[e] = f32_to_e2m1(ldexpf(c[e], -sexp));
    if constexpr (DPL == 1) {
      // two lanes share a byte: the even lane writes (own | neighbour << 4)
      uint32_t other = (uint32_t)__shfl_xor((int)nib[0], 1, 64);
      if ((lane & 1) == 0)
        out_rows[orow * (int64_t)(D / 2) + lane / 2] = (uint8_t)(nib[0] | (other << 4));
    } else {
#pragma unroll
      for (int e = 0; e < DPL / 2; e++) o[e] = (uint8_t)(nib[2 * e] | (nib[2 * e + 1] << 4));
    }
    if (lane % LPB == 0) out_scales[orow * (int64_t)(D / 32) + lane / LPB] = (uint8_t)(sexp + 127);
  }
}

template <int DPL, bool RAW_BF16, int WAVES, bool ROPE>
static hipError_t launch_waves(const KvCompressArgs& a) {
  const int64_t groups = (int64_t)a.B * a.G;
  dim3 grid((unsigned)(WAVES == 1 ? (groups + 3) / 4 : groups)), block(64 * (WAVES == 1 ? 4 : WAVES));
  hipStream_t s = (hipStream_t)a.stream;
  switch (a.out_fmt) {
    case CSAH_FMT_ROW_F32:
      a.prof.launch(kv_compress_kernel<DPL, RAW_BF16, CSAH_FMT_ROW_F32, WAVES, ROPE>, grid, block, s,
          a.raw, a.raw_seq_stride, a.B, a.G, a.m, a.span, a.skip, a.w, a.beta, (uint8_t*)a.out_rows,
          a.out_map, a.first_entry, a.out_scales, a.tok_pos, a.rope_dims,
          a.rope_base);
      break;
    case CSAH_FMT_ROW_E4M3_BF16:
      if constexpr (DPL == 8)
        a.prof.launch(kv_compress_kernel<DPL, RAW_BF16, CSAH_FMT_ROW_E4M3_BF16, WAVES, ROPE>, grid, block, s,
            a.raw, a.raw_seq_stride, a.B, a.G, a.m, a.span, a.skip, a.w, a.beta, (uint8_t*)a.out_rows,
            a.out_map, a.first_entry, a.out_scales, a.tok_pos, a.rope_dims,
          a.rope_base);
      else
        return hipErrorInvalidValue;
      break;
    default:
      a.prof.launch(kv_compress_kernel<DPL, RAW_BF16, CSAH_FMT_FP4_E8M0, WAVES, ROPE>, grid, block, s,
          a.raw, a.raw_seq_stride, a.B, a.G, a.m, a.span, a.skip, a.w, a.beta, (uint8_t*)a.out_rows,
          a.out_map, a.first_entry, a.out_scales, a.tok_pos, a.rope_dims,
          a.rope_base);
  }
  return hipGetLastError();
}

template <int DPL, bool RAW_BF16>
static hipError_t launch_dpl(const KvCompressArgs& a) {
  // a whole workgroup per entry once the span is long enough to keep 4 wavefronts busy, 8
  // wavefronts (two batches each for 128 tokens) past 8 batches
  if (a.rope_dims > 0)
    return a.span > 8 * kTokBatch   ? launch_waves<DPL, RAW_BF16, 8, true>(a)
           : a.span > 2 * kTokBatch ? launch_waves<DPL, RAW_BF16, 4, true>(a)
                                    : launch_waves<DPL, RAW_BF16, 1, true>(a);
  return a.span > 8 * kTokBatch   ? launch_waves<DPL, RAW_BF16, 8, false>(a)
         : a.span > 2 * kTokBatch ? launch_waves<DPL, RAW_BF16, 4, false>(a)
                                  : launch_waves<DPL, RAW_BF16, 1, false>(a);
}

template <bool RAW_BF16>
static hipError_t launch_raw(const KvCompressArgs& a) {
  switch (a.D) {
    case 64: return launch_dpl<1, RAW_BF16>(a);
    case 128: return launch_dpl<2, RAW_BF16>(a);
    case 256: return launch_dpl<4, RAW_BF16>(a);
    case 512: return launch_dpl<8, RAW_BF16>(a);
    case 1024: return launch_dpl<16, RAW_BF16>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kv_compress(const KvCompressArgs& a) {
  if (a.B == 0 || a.G == 0) return hipSuccess;
  return a.raw_dtype == CSAH_DT_BF16 ? launch_raw<true>(a) : launch_raw<false>(a);
}

}  // namespace csah
