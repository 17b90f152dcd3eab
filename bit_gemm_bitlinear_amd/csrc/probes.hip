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

int blprobe_mfma_i8(int64_t workgroups, int32_t iters, int32_t pattern, int32_t* sink,
                    void* stream) {
  if (!sink || workgroups < 1 || workgroups > (int64_t(1) << 20) || iters < 1 ||
      iters > (1 << 16) || (pattern != 0 && pattern != 1))
    return 1;
  mfma_loop_kernel<<<(unsigned)workgroups, kThreads, 0, (hipStream_t)stream>>>(iters, pattern, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
