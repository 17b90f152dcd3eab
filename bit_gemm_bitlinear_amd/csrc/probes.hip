// Measurement kernels of libbitlinear_probes.so (include/bitlinear_probes.h):
// the achievable memory-read rate and int8 matrix-core rate of the GPU, the
// ceilings that the decode and prefill contractions are measured against.
#include "../../include/bitlinear_probes.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
static_assert(kThreads == 256, "four partial results per workgroup");
constexpr int kReadWgsPerCu = 32;  // the fastest of the shapes tried (1 GiB: 6.7 TB/s)

// One 16-byte nontemporal load per thread and step of a grid-stride loop.
// Deeper unrolling and plain (temporal) loads both read slower.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const v4i* __restrict__ p, int64_t n16,
                                                               int32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  v4i acc = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    acc ^= __builtin_nontemporal_load(p + i);
  int32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  // one atomic per workgroup, spread over the sink words: device-scope
  // atomics on one word from every wave of the chip serialize
  __shared__ int32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicXor(sink + (blockIdx.x % BLPROBE_SINK_WORDS), part[0] ^ part[1] ^ part[2] ^ part[3]);
}

// A 32-bit mixing function (the finalizer of MurmurHash3).
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// Four bytes: activation-like (-127..127) or weight-code-like (0..2).
__device__ __forceinline__ int32_t rand_bytes(uint32_t key, bool codes) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t h = mix32(key * 4u + (uint32_t)b);
    const uint32_t v = codes ? h % 3u : (uint32_t)((int32_t)(h % 255u) - 127) & 0xFFu;
    r |= v << (8 * b);
  }
  return (int32_t)r;
}

__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, int pattern,
                                                             int32_t* __restrict__ sink) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  v4i a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = (t * 2u + (uint32_t)s) * 4u + (uint32_t)e;
      a[s][e] = pattern == 0 ? 0x01010101 : rand_bytes(key, false);
      b[s][e] = pattern == 0 ? 0x01010101 : rand_bytes(key ^ 0x5BD1E995u, true);
    }
  v16i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j & 1], b[j & 1], acc[j], 0, 0, 0);
  }
  uint32_t s = 0;  // wraps modulo 2^32 with random operands
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (uint32_t)acc[j][r];
  sink[t] = (int32_t)s;
}

// ---------------------------------------------------------------------------
// A lookup-table contraction for one token row (the idea of T-MAC, which the
// GeekNews page on bitnet.cpp names as the basis of its CPU kernels), kept as
// the alternative the matrix-core decode is measured against.  For every
// pair of activation codes (q[2j], q[2j+1]) the workgroup tabulates, in LDS,
// the 16 sums q[2j] (c0 - 1) + q[2j+1] (c1 - 1) over the 2-bit weight codes
// c0, c1 -- one 4-bit field of a packed byte indexes them.  The weights then
// cost one table read and one add per pair instead of a multiply-add each.
// Weights are read in the 16-row tiled layout (common.hpp of the library),
// the same 1 KB per wave load as the matrix-core decode: lane (r, g) holds
// packed bytes 16 g .. 16 g + 15 of row r in each 256-weight tile.
constexpr int kLutMaxK = 8192;
constexpr int kLutPartK = 2048;  // weights of a row per workgroup (table: 33 KB of LDS)
constexpr int kLutRing = 8;      // tiles in flight per lane

// Index (in int16 entries) of entry `nib` of pair j: 16 entries per pair and
// one pair of padding per 32, so that the four 32-pair runs that the four
// lane groups of a wave read fall on different LDS banks.
__device__ __forceinline__ int lut_index(int j, int nib) { return (j + (j >> 5)) * 16 + nib; }

__global__ __launch_bounds__(kThreads) void lut_zero_kernel(int32_t* __restrict__ acc, int n) {
  for (int i = (int)(blockIdx.x * kThreads + threadIdx.x); i < n; i += (int)(gridDim.x * kThreads))
    acc[i] = 0;
}

// Workgroup (b, p): 16-row blocks 4b .. 4b+3 (one per wave) over K part p
// (kLutPartK weights); partial sums are added to acc (exact integers, so the
// parts may land in any order).
__global__ __launch_bounds__(kThreads) void lut_decode_kernel(const int8_t* __restrict__ q, int k,
                                                              const uint8_t* __restrict__ tiled,
                                                              int n, int32_t* __restrict__ acc) {
  __shared__ __align__(16) int16_t tab[(kLutPartK / 2 + kLutPartK / 64) * 16];
  const int parts = (k + kLutPartK - 1) / kLutPartK;
  const int part = (int)blockIdx.x % parts, wgb = (int)blockIdx.x / parts;
  const int k0 = part * kLutPartK, kp = min(kLutPartK, k - k0);
  // the part's table: thread t builds pairs t, t + 256, ... with two 16-byte stores each
  for (int j = threadIdx.x; j < kp / 2; j += kThreads) {
    const int32_t a = q[k0 + 2 * j], b = q[k0 + 2 * j + 1];
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n0 = 2 * e, n1 = 2 * e + 1;
      const uint32_t lo = (uint16_t)(int16_t)(a * ((n0 & 3) - 1) + b * ((n0 >> 2) - 1));
      const uint32_t hi = (uint16_t)(int16_t)(a * ((n1 & 3) - 1) + b * ((n1 >> 2) - 1));
      h[e] = lo | (hi << 16);
    }
    v4i* dst = reinterpret_cast<v4i*>(tab + lut_index(j, 0));
    dst[0] = v4i{(int32_t)h[0], (int32_t)h[1], (int32_t)h[2], (int32_t)h[3]};
    dst[1] = v4i{(int32_t)h[4], (int32_t)h[5], (int32_t)h[6], (int32_t)h[7]};
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int blk = wgb * 4 + wave;
  if (blk >= (n >> 4)) return;
  const int tiles = kp >> 8;
  const int64_t rowbytes = k >> 2;
  const uint8_t* base = tiled + (int64_t)blk * 16 * rowbytes + 1024 * (int64_t)(k0 >> 8) + 16 * lane;
  int32_t sum = 0;
  for (int t0 = 0; t0 < tiles; t0 += kLutRing) {
    v4i w[kLutRing];
#pragma unroll
    for (int u = 0; u < kLutRing; ++u)
      w[u] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(base + 1024 * (int64_t)min(t0 + u, tiles - 1)));
#pragma unroll
    for (int u = 0; u < kLutRing; ++u) {
      if (t0 + u >= tiles) break;
      // pair 128 t + 32 g + 8 d + e (of the part) is nibble e of dword d of this chunk
      const int jb = 128 * (t0 + u) + 32 * g;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t x = (uint32_t)w[u][d];
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += tab[lut_index(jb + 8 * d + e, (x >> (4 * e)) & 15u)];
      }
    }
  }
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
  if (g == 0) atomicAdd(acc + blk * 16 + r, sum);
}

}  // namespace

extern "C" {

int blprobe_stream_read(const void* buf, int64_t bytes, int32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 5;
  const int64_t n16 = bytes / 16;
  int64_t grid = (int64_t)cus * kReadWgsPerCu;
  const int64_t need = (n16 + kThreads - 1) / kThreads;
  if (grid > need) grid = need;
  stream_read_kernel<<<(unsigned)grid, kThreads, 0, (hipStream_t)stream>>>(
      reinterpret_cast<const v4i*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int blprobe_lut_decode_acc(const int8_t* q, int64_t k, const uint8_t* tiled, int64_t n,
                           int32_t* acc, void* stream) {
  if (!q || !tiled || !acc || k < 256 || k > kLutMaxK || k % 256 != 0 || n < 16 || n % 16 != 0 ||
      n > (int64_t(1) << 26) || ((uintptr_t)q & 15) || ((uintptr_t)tiled & 15) || ((uintptr_t)acc & 15))
    return 1;
  const hipStream_t s = (hipStream_t)stream;
  lut_zero_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(acc, (int)n);
  const int64_t parts = (k + kLutPartK - 1) / kLutPartK;
  const int64_t grid = (n / 16 + 3) / 4 * parts;
  lut_decode_kernel<<<(unsigned)grid, kThreads, 0, s>>>(q, (int)k, tiled, (int)n, acc);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int blprobe_mfma_i8(int64_t workgroups, int32_t iters, int32_t pattern, int32_t* sink,
                    void* stream) {
  if (!sink || workgroups < 1 || workgroups > (int64_t(1) << 20) || iters < 1 ||
      iters > (1 << 16) || (pattern != 0 && pattern != 1))
    return 1;
  mfma_loop_kernel<<<(unsigned)workgroups, kThreads, 0, (hipStream_t)stream>>>(iters, pattern, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
