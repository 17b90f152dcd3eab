// Decode contraction (M <= 16 tokens): acc[m][n] = sum_k q[m][k] * u[n][k],
// then y = bf16(acc / (x_scale[m] * w_scale)) -- the F.linear call and
// post_quant_process of BitLinear.forward in the Falcon-Edge blog ("A series
// of powerful, universal and fine-tunable 1.58-bit language models", section
// "Falcon-Edge, a series of universal models"), in exact integer arithmetic.
//
// This is bound by HBM bandwidth on the packed weights (2 bits per weight),
// so the kernel is organised around streaming them once:
//  * work unit: a workgroup (4 waves) owns 16*TW consecutive weight rows and
//    a range of K (all of it unless K is split for LDS space); every lane
//    issues all of its 16-byte weight loads before touching anything else,
//    so a whole decoder layer is in flight at once;
//  * the activation codes (int8, prepared by act_quant.hip) are staged once
//    per workgroup in LDS;
//  * each 16 packed bytes hold 64 weights = four K-steps of one row for the
//    16x16x64 int8 matrix-core op; they are expanded in registers to codes
//    c = u + 1 with one shift and one mask per dword (common.hpp), and
//    sum q*u = sum q*c - sum q is restored with the per-row code sum;
//  * token rows m >= M of the 16-row A operand are zeros (no LDS reads);
//  * the four waves split K, and their partial sums meet in LDS.
// Loads past the end of a row or past the last row are clamped to valid
// addresses instead of masked: the activation codes there are zero (rows of
// codes are zero-padded) and output columns of rows >= N are never stored.
#include "common.hpp"
#include "internal.hpp"

namespace bl {

namespace {

constexpr int kThreads = 256;
constexpr int kStageUnits = kDecodeLdsA / 16 / kThreads;  // 16-byte A units per thread

// 16 bytes of a packed row at byte offset `off` (a multiple of 16).  Parts
// past `rowbytes` read the row's last bytes instead (multiplied by zero).
// MODE 0: rowbytes % 16 == 0 (one 128-bit load); 1: rowbytes % 4 == 0;
// 2: any length.  A compile-time choice keeps the loads branch-free.
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

template <int TW, int MODE>
__device__ __forceinline__ void decode_body(const DecodeArgs& A, const DecodeProj& P, int wl,
                                            int8_t* __restrict__ lds, int* __restrict__ flag) {
  constexpr int MAXS = decode_max_items(MODE) / TW;  // slabs per wave held in registers
  const int M = A.m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int group = wl / P.ksplit, kpart = wl - group * P.ksplit;
  const int row0 = group * 16 * TW;
  const int S = (P.k + 255) >> 8;
  const int sb = kpart * P.kspw;
  const int ns = min(S, sb + P.kspw) - sb;  // slabs of this WG
  const int nsw = (ns + 3) >> 2;            // slabs per wave
  const int ws0 = min(ns, wave * nsw);
  const int nw = min(ns, ws0 + nsw) - ws0;  // slabs of this wave (may be 0)
  const int rowbytes = P.k >> 2;
  const int lrow = A.lds_row;

  // 1. activation codes of this WG -> registers (issued first: L2 hits)
  const int upr = ns * 16;  // 16-byte units per token row
  const int units = M * upr;
  v4i stage[kStageUnits];
#pragma unroll
  for (int i = 0; i < kStageUnits; ++i) {
    int u = min((int)threadIdx.x + kThreads * i, units - 1);
    int m = u / upr, c = u - m * upr;
    stage[i] = *reinterpret_cast<const v4i*>(P.q + (int64_t)m * P.ldq + sb * 256 + c * 16);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. every weight load of this lane, in consumption order
  v4i breg[MAXS][TW];
  const int lsmax = max(nw - 1, 0);
#pragma unroll
  for (int ls = 0; ls < MAXS; ++ls) {
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int row = min(row0 + 16 * t + ln, P.n - 1);
      const int slab = sb + ws0 + min(ls, lsmax);
      breg[ls][t] = load_w16<MODE>(P.packed + (int64_t)row * rowbytes, slab * 64 + 16 * lg,
                                   rowbytes);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. staged codes -> LDS
#pragma unroll
  for (int i = 0; i < kStageUnits; ++i) {
    int u = (int)threadIdx.x + kThreads * i;
    if (u < units) {
      int m = u / upr, c = u - m * upr;
      *reinterpret_cast<v4i*>(lds + m * lrow + c * 16) = stage[i];
    }
  }
  __syncthreads();

  // 4. contraction: per slab, the four A fragments feed TW row tiles
  v4i acc[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) acc[t] = v4i{0, 0, 0, 0};
  const bool live = ln < M;
  const int8_t* abase = lds + (live ? ln : 0) * lrow + 64 * lg;
#pragma unroll
  for (int ls = 0; ls < MAXS; ++ls) {
    if (ls < nw) {
      v4i a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v4i v = *reinterpret_cast<const v4i*>(abase + (ws0 + ls) * 256 + 16 * j);
        a[j] = live ? v : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < TW; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[t] = mfma_16x16x64_i8(a[j], decode16((uint32_t)breg[ls][t][j]), acc[t]);
      }
    }
  }
  __syncthreads();  // LDS is reused below

  // 5. cross-wave reduction: red[wave][t][m][16]; lane holds rows 4*lg+r, column ln
  int32_t* red = reinterpret_cast<int32_t*>(lds);
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lg + r;
      if (m < M) red[((wave * TW + t) * M + m) * 16 + ln] = acc[t][r];
    }
  }
  __syncthreads();

  const int nout = TW * M * 16;
  const int wstride = TW * M * 16;
  if (P.ksplit == 1) {
    const float ws = P.y ? P.w_scale[0] : 0.0f;
    for (int idx = threadIdx.x; idx < nout; idx += kThreads) {
      const int t = idx / (M * 16), rem = idx - t * M * 16, m = rem >> 4, c = rem & 15;
      const int n = row0 + 16 * t + c;
      if (n >= P.n) continue;
      const int32_t v = red[idx] + red[idx + wstride] + red[idx + 2 * wstride] +
                        red[idx + 3 * wstride] - P.qsum[m];
      if (P.y)
        P.y[(int64_t)m * P.n + n] = dequant_bf16(v, P.x_scale[m], ws);
      else
        P.acc_out[(int64_t)m * P.n + n] = v;
    }
    return;
  }

  // K split across WGs: add partials in L2, the last WG of the row group
  // finishes (integer addition, so the arrival order does not matter).
  for (int idx = threadIdx.x; idx < nout; idx += kThreads) {
    const int t = idx / (M * 16), rem = idx - t * M * 16, m = rem >> 4, c = rem & 15;
    const int n = row0 + 16 * t + c;
    if (n >= P.n) continue;
    atomicAdd(&P.part[(int64_t)m * P.n + n],
              red[idx] + red[idx + wstride] + red[idx + 2 * wstride] + red[idx + 3 * wstride]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) *flag = (atomicAdd(&P.count[group], 1u) == (uint32_t)(P.ksplit - 1));
  __syncthreads();
  if (!*flag) return;
  __threadfence();
  const float ws = P.y ? P.w_scale[0] : 0.0f;
  for (int idx = threadIdx.x; idx < nout; idx += kThreads) {
    const int t = idx / (M * 16), rem = idx - t * M * 16, m = rem >> 4, c = rem & 15;
    const int n = row0 + 16 * t + c;
    if (n >= P.n) continue;
    const int32_t v = atomicAdd(&P.part[(int64_t)m * P.n + n], 0) - P.qsum[m];
    if (P.y)
      P.y[(int64_t)m * P.n + n] = dequant_bf16(v, P.x_scale[m], ws);
    else
      P.acc_out[(int64_t)m * P.n + n] = v;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeArgs A) {
  extern __shared__ __align__(16) int8_t lds[];
  __shared__ int flag;
  int pi = 0;
  while (pi + 1 < A.count && (int)blockIdx.x >= A.p[pi + 1].wg_begin) ++pi;
  const DecodeProj& P = A.p[pi];
  const int wl = (int)blockIdx.x - P.wg_begin;
  constexpr int kMaxTw = decode_max_items(MODE) < kDecodeMaxTw ? decode_max_items(MODE)
                                                                : kDecodeMaxTw;
  switch (P.tw) {
    case 1: decode_body<1, MODE>(A, P, wl, lds, &flag); break;
    case 2: decode_body<2, MODE>(A, P, wl, lds, &flag); break;
    case 3: if constexpr (kMaxTw >= 3) decode_body<3, MODE>(A, P, wl, lds, &flag); break;
    case 4: if constexpr (kMaxTw >= 4) decode_body<4, MODE>(A, P, wl, lds, &flag); break;
    case 5: if constexpr (kMaxTw >= 5) decode_body<5, MODE>(A, P, wl, lds, &flag); break;
    case 6: if constexpr (kMaxTw >= 6) decode_body<6, MODE>(A, P, wl, lds, &flag); break;
    case 7: if constexpr (kMaxTw >= 7) decode_body<7, MODE>(A, P, wl, lds, &flag); break;
    case 8: if constexpr (kMaxTw >= 8) decode_body<8, MODE>(A, P, wl, lds, &flag); break;
    default: break;
  }
}

}  // namespace

// Choose the work split of one projection: K per WG limited by the LDS
// budget for staged codes and by the register budget (16 loads per lane),
// then as many 16-row tiles per WG as fill the register budget (so every
// lane issues about 16 loads of 16 bytes and a WG moves about 64 KB).
DecodePlan plan_decode(int64_t m, int64_t n, int64_t k, int mode) {
  DecodePlan p;
  const int items = decode_max_items(mode);
  const int S = (int)((k + 255) / 256);
  int cap_lds = (int)((kDecodeLdsA / m - 16) / 256);
  if (cap_lds < 1) cap_lds = 1;
  const int cap = cap_lds < 4 * items ? cap_lds : 4 * items;
  p.ksplit = (S + cap - 1) / cap;
  p.kspw = (S + p.ksplit - 1) / p.ksplit;
  const int nsw = (p.kspw + 3) / 4;
  int tw = items / nsw;
  if (tw > kDecodeMaxTw) tw = kDecodeMaxTw;
  if (tw < 1) tw = 1;
  const int tiles = (int)((n + 15) / 16);
  if (tw > tiles) tw = tiles;
  p.tw = tw;
  p.ngroups = (int)((n + 16 * tw - 1) / (16 * tw));
  return p;
}

size_t decode_lds_bytes(int64_t m, const DecodePlan& p) {
  size_t a = (size_t)m * ((size_t)p.kspw * 256 + 16);
  size_t r = (size_t)4 * p.tw * m * 16 * 4;
  return a > r ? a : r;
}

hipError_t launch_decode(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s) {
  if (a.load_mode == 0)
    decode_kernel<0><<<(unsigned)total_wgs, kThreads, lds_bytes, s>>>(a);
  else if (a.load_mode == 1)
    decode_kernel<1><<<(unsigned)total_wgs, kThreads, lds_bytes, s>>>(a);
  else
    decode_kernel<2><<<(unsigned)total_wgs, kThreads, lds_bytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace bl
