// Weight preparation: the Falcon-Edge blog's _weight_quant ("A series of
// powerful, universal and fine-tunable 1.58-bit language models", section
// "Falcon-Edge, a series of universal models") followed by 2-bit storage.
//
//   scale = 1 / max(mean|w|, 1e-5);  u = clamp(round(w * scale), -1, 1)
//
// mean|w| must not depend on how the sum is split across threads, or the
// ternary codes of large tensors would change from run to run.  The sum is
// therefore exact: every |w| is m * 2^(max(E,1) - 150) with a 24-bit
// significand m and biased exponent E, so adding the significands per
// exponent in 64-bit integers loses nothing (atomics included, since
// integer addition is associative).  One thread then forms the exact total
// and divides by the element count, rounding once to fp32
// (absmean_round.hpp).  Four small launches, no host synchronization; the
// scale stays on the device.
#include "absmean_round.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace bl {

namespace {

constexpr int kBuckets = 256;

__global__ void zero_buckets_kernel(unsigned long long* b) {
  b[threadIdx.x] = 0ull;
}

__device__ __forceinline__ void bucket_add(unsigned long long* h, float v) {
  uint32_t bits = __float_as_uint(v) & 0x7FFFFFFFu;
  uint32_t e = bits >> 23;
  uint32_t m = (bits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  if (m) atomicAdd(&h[e], (unsigned long long)m);
}

// Per-wave LDS histograms (less contention), merged into the global one.
__global__ __launch_bounds__(256) void absmean_hist_kernel(const float* __restrict__ w,
                                                           int64_t count,
                                                           unsigned long long* __restrict__ out) {
  __shared__ unsigned long long h[4][kBuckets];
  for (int i = threadIdx.x; i < 4 * kBuckets; i += blockDim.x) (&h[0][0])[i] = 0ull;
  __syncthreads();
  unsigned long long* mine = h[threadIdx.x >> 6];
  const int64_t n4 = count >> 2;
  const float4* w4 = reinterpret_cast<const float4*>(w);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 v = w4[i];
    bucket_add(mine, v.x);
    bucket_add(mine, v.y);
    bucket_add(mine, v.z);
    bucket_add(mine, v.w);
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += stride)
    bucket_add(mine, w[i]);
  __syncthreads();
  for (int e = threadIdx.x; e < kBuckets; e += blockDim.x) {
    unsigned long long v = h[0][e] + h[1][e] + h[2][e] + h[3][e];
    if (v) atomicAdd(&out[e], v);
  }
}

// One thread: exact mean (absmean_round.hpp), then w_scale = 1 / max(mean, 1e-5).
__global__ void absmean_finalize_kernel(const unsigned long long* __restrict__ buckets,
                                        uint64_t count, float* __restrict__ w_scale) {
  if (threadIdx.x != 0) return;
  const float mean = __uint_as_float(absmean_bits_from_buckets(buckets, count));
  w_scale[0] = 1.0f / fmaxf(mean, kEps);
}

// Byte i of the flattened [N][K/4] output holds flattened weights 4i..4i+3
// (K % 4 == 0, so a byte never straddles two rows).
__global__ __launch_bounds__(256) void ternarize_pack_kernel(const float* __restrict__ w,
                                                             int64_t nbytes,
                                                             const float* __restrict__ w_scale,
                                                             uint8_t* __restrict__ packed) {
  const float s = w_scale[0];
  const float4* w4 = reinterpret_cast<const float4*>(w);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nbytes; i += stride) {
    float4 v = w4[i];
    uint32_t b = ternary_code(v.x, s) | (ternary_code(v.y, s) << 2) |
                 (ternary_code(v.z, s) << 4) | (ternary_code(v.w, s) << 6);
    packed[i] = (uint8_t)b;
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                     int64_t nbytes, int8_t* __restrict__ u) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nbytes; i += stride) {
    uint32_t b = packed[i];
    uint32_t c = (b & 3u) | (((b >> 2) & 3u) << 8) | (((b >> 4) & 3u) << 16) |
                 (((b >> 6) & 3u) << 24);
    // per-byte c - 1 without borrows: add 0xFF (== -1 mod 256) to each byte
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) out |= (((c >> (8 * j)) + 0xFFu) & 0xFFu) << (8 * j);
    reinterpret_cast<uint32_t*>(u)[i] = out;
  }
}

// Row-major <-> tiled layout (common.hpp): one 16-byte chunk per thread and
// step, walked in the order of the tiled bytes.  A block of 16 rows holds
// rowbytes chunks; chunk u of a block is row u % 16, chunk (u / 16) % 4 of
// that row's 64 bytes in tile u / 64.
__global__ __launch_bounds__(256) void tile_kernel(const uint8_t* __restrict__ src, int64_t chunks,
                                                   int64_t rowbytes, uint8_t* __restrict__ dst,
                                                   int untile) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < chunks; d += stride) {
    const int64_t blk = d / rowbytes, u = d - blk * rowbytes;
    const int64_t row = 16 * blk + (u & 15);
    const int64_t rowpos = row * rowbytes + 64 * (u >> 6) + 16 * ((u >> 4) & 3);
    const int64_t from = untile ? 16 * d : rowpos, to = untile ? rowpos : 16 * d;
    *G(reinterpret_cast<v4i*>(dst + to)) = *G(reinterpret_cast<const v4i*>(src + from));
  }
}

// The "universal" bf16 export: u / w_scale for every weight (the blog's
// state_dict loop after _weight_quant), from the packed codes.  The four
// possible values (codes 0..3, u = -1, 0, 1, 2) are one fp32 division each,
// rounded to bf16, computed once per thread.  Thread work: one 16-byte chunk
// of a packed row (64 weights) in either layout -> 128 bytes of row-major
// bf16 output.
__global__ __launch_bounds__(256) void export_bf16_kernel(const uint8_t* __restrict__ packed,
                                                          int64_t chunks, int64_t rowbytes,
                                                          int tiled, const float* __restrict__ w_scale,
                                                          uint16_t* __restrict__ out) {
  const float s = load_f32_vmem(w_scale);
  uint32_t lut[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) lut[c] = f32_to_bf16((float)(c - 1) / s);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t cpr = rowbytes >> 4;  // chunks per row
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += stride) {
    const int64_t row = i / cpr, o = 16 * (i - row * cpr);
    const int64_t src = tiled ? tiled_chunk_offset(row, o, rowbytes) : row * rowbytes + o;
    const v4i p = *G(reinterpret_cast<const v4i*>(packed + src));
    v4i* dst = reinterpret_cast<v4i*>(out + row * (rowbytes * 4) + 4 * o);
#pragma unroll
    for (int d = 0; d < 4; ++d) {  // dword d: weights 16d .. 16d+15
      const uint32_t w = (uint32_t)p[d];
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t c0 = (w >> (4 * j)) & 3u, c1 = (w >> (4 * j + 2)) & 3u;
        h[j] = lut[c0] | (lut[c1] << 16);
      }
      *G(dst + 2 * d) = v4i{(int32_t)h[0], (int32_t)h[1], (int32_t)h[2], (int32_t)h[3]};
      *G(dst + 2 * d + 1) = v4i{(int32_t)h[4], (int32_t)h[5], (int32_t)h[6], (int32_t)h[7]};
    }
  }
}

// Rows whose packed length is not a multiple of 16 (K % 64 != 0, row-major
// only): one packed byte per thread.
__global__ __launch_bounds__(256) void export_bf16_bytes_kernel(const uint8_t* __restrict__ packed,
                                                                int64_t nbytes,
                                                                const float* __restrict__ w_scale,
                                                                uint16_t* __restrict__ out) {
  const float s = load_f32_vmem(w_scale);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nbytes; b += stride) {
    // row-major: byte b of the flattened [n][k/4] array holds weights 4b..4b+3
    const uint32_t w = packed[b];
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * b + j] = f32_to_bf16((float)((int)((w >> (2 * j)) & 3u) - 1) / s);
  }
}

int grid_for(int64_t work, int per_block, int cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

}  // namespace

hipError_t launch_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* w_scale,
                       unsigned long long* buckets, hipStream_t s) {
  const int64_t count = n * k;
  zero_buckets_kernel<<<1, kBuckets, 0, s>>>(buckets);
  absmean_hist_kernel<<<grid_for(count / 4, 256 * 8, 4096), 256, 0, s>>>(w, count, buckets);
  absmean_finalize_kernel<<<1, 64, 0, s>>>(buckets, (uint64_t)count, w_scale);
  const int64_t nbytes = count / 4;
  ternarize_pack_kernel<<<grid_for(nbytes, 256 * 4, 8192), 256, 0, s>>>(w, nbytes, w_scale,
                                                                        packed);
  return hipGetLastError();
}

hipError_t launch_tile(const uint8_t* src, int64_t n, int64_t k, uint8_t* dst, bool untile,
                       hipStream_t s) {
  const int64_t chunks = n * k / 64;
  tile_kernel<<<grid_for(chunks, 256 * 4, 8192), 256, 0, s>>>(src, chunks, k / 4, dst,
                                                              untile ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_export_bf16(const uint8_t* packed, int64_t n, int64_t k, bool tiled,
                              const float* w_scale, uint16_t* out, hipStream_t s) {
  const int64_t rowbytes = k / 4;
  if (rowbytes % 16 == 0) {  // whole 16-byte chunks (always so in the tiled layout)
    const int64_t chunks = n * (rowbytes / 16);
    export_bf16_kernel<<<grid_for(chunks, 256 * 2, 8192), 256, 0, s>>>(packed, chunks, rowbytes,
                                                                       tiled ? 1 : 0, w_scale, out);
  } else {  // other row lengths (row-major only): byte by byte
    export_bf16_bytes_kernel<<<grid_for(n * rowbytes, 256 * 4, 8192), 256, 0, s>>>(
        packed, n * rowbytes, w_scale, out);
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* u, hipStream_t s) {
  const int64_t nbytes = n * k / 4;
  unpack_kernel<<<grid_for(nbytes, 256 * 4, 8192), 256, 0, s>>>(packed, nbytes, u);
  return hipGetLastError();
}

}  // namespace bl
