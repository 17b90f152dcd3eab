// Prefill contraction (M > 16 tokens) on the int8 matrix cores:
// acc[m][n] = sum_k q[m][k] * u[n][k], then y = bf16(acc / (x_scale[m] *
// w_scale)) -- F.linear and post_quant_process of BitLinear.forward in the
// Falcon-Edge blog ("A series of powerful, universal and fine-tunable 1.58-bit
// language models", section "Falcon-Edge, a series of universal models").
//
// A dense contraction, so it runs on v_mfma_i32_16x16x64_i8.  A workgroup
// computes a 128x128 output tile with four waves (2x2, 64x64 each).  Per
// 256-wide K slab a lane loads, for each of its four 16-column weight tiles,
// 16 packed bytes (64 weights = four K-steps of one row) and expands them in
// registers (common.hpp); the activation codes come from the internal layout
// written by act_quant.hip (rows padded to the tile, K padded to 256 with
// zero codes), so no operand load needs a bounds check.  Out-of-range weight
// rows and columns are clamped to valid addresses: they only reach output
// entries that are not stored, or meet zero activation codes.
#include "common.hpp"
#include "internal.hpp"

namespace bl {

namespace {

constexpr int kThreads = 256;

// 16 bytes of a packed row (see decode.hip); MODE fixes the row alignment.
template <int MODE>
__device__ __forceinline__ v4i load_w16(const uint8_t* __restrict__ row, int off, int rowbytes) {
  v4i r;
  if constexpr (MODE == 0) {
    r = *reinterpret_cast<const v4i*>(row + min(off, rowbytes - 16));
  } else if constexpr (MODE == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = *reinterpret_cast<const int32_t*>(row + min(off + 4 * j, rowbytes - 4));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t d = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) d |= (uint32_t)row[min(off + 4 * j + b, rowbytes - 1)] << (8 * b);
      r[j] = (int32_t)d;
    }
  }
  return r;
}

struct Frags {
  v4i a[4][4];  // [m tile][k step]
  v4i b[4];     // [n tile], 4 K-steps each
};

template <int MODE>
__device__ __forceinline__ void load_frags(Frags& f, const PrefillProj& P, int m0, int n0,
                                           int slab, int ln, int lg) {
  const int rowbytes = P.k >> 2;
#pragma unroll
  for (int nf = 0; nf < 4; ++nf) {
    const int row = min(n0 + 16 * nf + ln, P.n - 1);
    f.b[nf] = load_w16<MODE>(P.packed + (int64_t)row * rowbytes, slab * 64 + 16 * lg, rowbytes);
  }
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
    const int8_t* ap = P.q + (int64_t)(m0 + 16 * mf + ln) * P.ldq + slab * 256 + 64 * lg;
#pragma unroll
    for (int j = 0; j < 4; ++j) f.a[mf][j] = *reinterpret_cast<const v4i*>(ap + 16 * j);
  }
}

__device__ __forceinline__ void mma_slab(v4i (&acc)[4][4], const Frags& f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const v4i bj = decode16((uint32_t)f.b[nf][j]);
#pragma unroll
      for (int mf = 0; mf < 4; ++mf) acc[mf][nf] = mfma_16x16x64_i8(f.a[mf][j], bj, acc[mf][nf]);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillArgs A) {
  int pi = 0;
  while (pi + 1 < A.count && (int)blockIdx.x >= A.p[pi + 1].tile_begin) ++pi;
  const PrefillProj& P = A.p[pi];
  const int tl = (int)blockIdx.x - P.tile_begin;
  const int tm = tl % A.tiles_m, tn = tl / A.tiles_m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int m0 = tm * kPrefillBM + (wave & 1) * 64;
  const int n0 = tn * kPrefillBN + (wave >> 1) * 64;
  const int S = (P.k + 255) >> 8;

  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  Frags f0, f1;
  load_frags<MODE>(f0, P, m0, n0, 0, ln, lg);
  int s = 0;
  for (; s + 2 <= S; s += 2) {
    load_frags<MODE>(f1, P, m0, n0, s + 1, ln, lg);
    mma_slab(acc, f0);
    if (s + 2 < S) load_frags<MODE>(f0, P, m0, n0, s + 2, ln, lg);
    mma_slab(acc, f1);
  }
  if (s < S) mma_slab(acc, f0);

  const float ws = P.y ? P.w_scale[0] : 0.0f;
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mf + 4 * lg + r;
      if (m >= A.m) continue;
      const int32_t qs = P.qsum[m];
      const float xs = P.y ? P.x_scale[m] : 0.0f;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int n = n0 + 16 * nf + ln;
        if (n >= P.n) continue;
        const int32_t v = acc[mf][nf][r] - qs;
        if (P.y)
          P.y[(int64_t)m * P.n + n] = dequant_bf16(v, xs, ws);
        else
          P.acc_out[(int64_t)m * P.n + n] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int total_tiles, hipStream_t s) {
  if (a.load_mode == 0)
    prefill_kernel<0><<<(unsigned)total_tiles, kThreads, 0, s>>>(a);
  else if (a.load_mode == 1)
    prefill_kernel<1><<<(unsigned)total_tiles, kThreads, 0, s>>>(a);
  else
    prefill_kernel<2><<<(unsigned)total_tiles, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bl
