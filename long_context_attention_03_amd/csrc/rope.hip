// rope.hip -- RoPE on the rotary dims of query or output rows, in place.
//
// [BSWEN] "How DeepSeek V4 Handles 1M Token Context with Hybrid Attention", section "Component 1:
// Shared Key-Value Vectors": keys and values are one shared vector, and an inverse RoPE gives the
// attention result back its positional meaning. [EXPL] "Key numbers" (KV storage precision row):
// the rotary dims of a row are its BF16 part. The rotation is RoFormer's general form (Su et al.,
// "RoFormer: Enhanced Transformer with Rotary Position Embedding", section 3.2): the last R dims
// of a row are R/2 adjacent pairs, pair j turns by p * base^(-2j/R) at position p.
//
// One workgroup per (sequence, query) row group: its threads first compute the R/2 (cos, sin)
// pairs of the row group's position in fp64 into LDS, then turn every head's rotary pairs in
// fp64 and round once to the row's type (nearest, ties to even). Only the rotary dims are read
// and written. rope_vec_kernel moves whole 16-byte vectors when the rotary part allows it;
// rope_kernel takes one pair per thread for any other even width.
#include "csah_internal.h"
#include "device_common.h"

namespace csah {

// bf16 bits of v, rounded once from fp64 (nearest, ties to even): v is first rounded to 8
// significant bits in fp64 (exact; the bf16 subnormal spacing 2^-133 below 2^-126), which binary32
// then holds exactly, so its top half is the answer. A direct fp64 -> fp32 -> bf16 chain could
// round twice.
__device__ __noinline__ uint32_t f64_to_bf16_bits_slow(double v) {
  if (v == 0.0 || !(fabs(v) < INFINITY)) return f2u((float)v) >> 16 | (v != v ? 0x40u : 0u);
  int e = ilogb(v);
  if (e < -126) e = -126;
  const double r = ldexp(rint(ldexp(v, 7 - e)), e - 7);
  return f2u((float)r) >> 16;  // |r| >= 2^128 overflows to infinity, as rounding to bf16 does
}

// The same rounding on the binary64 pattern for |v| in the bf16 normal range: keeping the top 7 of
// the 52 stored significand bits, nearest with ties to even, is one integer add (a carry out of
// the significand moves the exponent up, as it should); the kept value then converts to binary32
// exactly.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t ex = (uint32_t)(u >> 52) & 0x7FFu;  // biased binary64 exponent
  if (ex < 1023 - 126 || ex == 0x7FFu) return f64_to_bf16_bits_slow(v);  // tiny, inf or NaN
  const uint64_t r = (u + 0x0FFFFFFFFFFFull + ((u >> 45) & 1u)) & ~0x1FFFFFFFFFFFull;
  return f2u((float)__builtin_bit_cast(double, r)) >> 16;
}

template <bool BF16>
__global__ __launch_bounds__(256) void rope_kernel(void* __restrict__ x, int Q, int H, int D,
                                                   int R, const int64_t* __restrict__ pos,
                                                   double base, int inverse) {
  __shared__ double cs[2 * kRopeMaxPairs];
  const int row = blockIdx.x;  // sequence b, query i
  const int b = row / Q, i = row - b * Q;
  const double p = (double)(pos[b] + i);
  const int np = R / 2;
  for (int j = threadIdx.x; j < np; j += blockDim.x)
    rope_cos_sin(p, j, R, base, inverse != 0, cs[2 * j], cs[2 * j + 1]);
  __syncthreads();
  const int64_t first = (int64_t)row * H * D + (D - R);  // element index of head 0's first pair
  for (int t = threadIdx.x; t < H * np; t += blockDim.x) {
    const int h = t / np, j = t - h * np;
    const int64_t e = first + (int64_t)h * D + 2 * j;
    const double c = cs[2 * j], s = cs[2 * j + 1];
    if constexpr (BF16) {
      uint32_t* px = (uint32_t*)((uint16_t*)x + e);  // 4-byte aligned: e is even
      const uint32_t w = *px;
      const double x0 = u2f(w << 16), x1 = u2f(w & 0xFFFF0000u);
      *px = f64_to_bf16_bits(x0 * c - x1 * s) | (f64_to_bf16_bits(x0 * s + x1 * c) << 16);
    } else {
      f32x2* px = (f32x2*)((float*)x + e);  // 8-byte aligned: e is even
      const f32x2 w = *px;
      const double x0 = w[0], x1 = w[1];
      *px = f32x2{(float)(x0 * c - x1 * s), (float)(x0 * s + x1 * c)};
    }
  }
}

// The same rotation when each head's rotary part is a whole number of 16-byte vectors starting on
// a 16-byte boundary ((D - R) and R multiples of 8 bf16 or 4 f32 values): a thread takes whole
// vectors, and issues the loads of its vectors (up to kRopeBatch per round) before turning any, so
// a row group costs one memory round trip per round instead of one per pair.
constexpr int kRopeBatch = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void rope_vec_kernel(void* __restrict__ x, int Q, int H, int D,
                                                       int R, const int64_t* __restrict__ pos,
                                                       double base, int inverse) {
  constexpr int VEC = BF16 ? 8 : 4;  // values per 16-byte vector
  __shared__ double cs[2 * kRopeMaxPairs];
  const int row = blockIdx.x;
  const int b = row / Q, i = row - b * Q;
  const int vph = R / VEC;  // vectors per head
  const int nvec = H * vph;
  const int64_t first = (int64_t)row * H * D + (D - R);
  u32x4 v[kRopeBatch];
  int64_t at[kRopeBatch];
  int j0[kRopeBatch];
  auto load_round = [&](int t0) {
#pragma unroll
    for (int u = 0; u < kRopeBatch; u++) {
      const int t = t0 + u * (int)blockDim.x;
      const int h = t / vph, k = t - h * vph;
      at[u] = first + (int64_t)h * D + (int64_t)k * VEC;
      j0[u] = k * (VEC / 2);
      if (t < nvec) {
        if constexpr (BF16)
          v[u] = *(const u32x4*)((const uint16_t*)x + at[u]);
        else
          v[u] = *(const u32x4*)((const float*)x + at[u]);
      }
    }
  };
  // the first round's loads go out before the table, so their latency covers the sines
  load_round(threadIdx.x);
  const double p = (double)(pos[b] + i);
  for (int j = threadIdx.x; j < R / 2; j += blockDim.x)
    rope_cos_sin(p, j, R, base, inverse != 0, cs[2 * j], cs[2 * j + 1]);
  __syncthreads();
  for (int t0 = threadIdx.x; t0 < nvec; t0 += kRopeBatch * blockDim.x) {
    if (t0 != (int)threadIdx.x) load_round(t0);
#pragma unroll
    for (int u = 0; u < kRopeBatch; u++) {
      if (t0 + u * (int)blockDim.x >= nvec) break;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < VEC / 2; e++) {
        const double c = cs[2 * (j0[u] + e)], sn = cs[2 * (j0[u] + e) + 1];
        if constexpr (BF16) {
          const uint32_t pr = v[u][e];
          const double x0 = u2f(pr << 16), x1 = u2f(pr & 0xFFFF0000u);
          w[e] = f64_to_bf16_bits(x0 * c - x1 * sn) | (f64_to_bf16_bits(x0 * sn + x1 * c) << 16);
        } else {
          const double x0 = u2f(v[u][2 * e]), x1 = u2f(v[u][2 * e + 1]);
          w[2 * e] = f2u((float)(x0 * c - x1 * sn));
          w[2 * e + 1] = f2u((float)(x0 * sn + x1 * c));
        }
      }
      if constexpr (BF16)
        *(u32x4*)((uint16_t*)x + at[u]) = w;
      else
        *(u32x4*)((float*)x + at[u]) = w;
    }
  }
}

hipError_t launch_rope(const RopeArgs& a) {
  if (a.B == 0 || a.Q == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.B * a.Q)), block(256);
  hipStream_t s = (hipStream_t)a.stream;
  const int vec = a.dtype == CSAH_DT_BF16 ? 8 : 4;
  const bool whole = a.R % vec == 0 && (a.D - a.R) % vec == 0;
  if (a.dtype == CSAH_DT_BF16)
    a.prof.launch(whole ? rope_vec_kernel<true> : rope_kernel<true>, grid, block, s, a.x, a.Q,
                  a.H, a.D, a.R, a.pos, a.base, a.inverse);
  else
    a.prof.launch(whole ? rope_vec_kernel<false> : rope_kernel<false>, grid, block, s, a.x, a.Q,
                  a.H, a.D, a.R, a.pos, a.base, a.inverse);
  return hipGetLastError();
}

}  // namespace csah
