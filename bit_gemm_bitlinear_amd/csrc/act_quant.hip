// Per-token activation quantization: the Falcon-Edge blog's
// activation_norm_quant ("A series of powerful, universal and fine-tunable
// 1.58-bit language models", section "Falcon-Edge, a series of universal
// models"):  scale = 127 / max(max_k |x|, 1e-5);  q = clamp(round(x*scale),
// -128, 127).  One workgroup per row: an integer max over the bf16 magnitude
// bits (exact), then one fp32 division and one multiply + round per code.
//
// Two outputs: the public natural layout [M][K], and the internal layout the
// contraction kernels read (rows padded with zero codes to a multiple of 256,
// each group of 16 codes stored 4x4-transposed to match the weight decode in
// common.hpp, plus the per-row code sum used to turn unsigned weight codes
// c = u + 1 back into u: sum q*u = sum q*c - sum q).
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace bl {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

__device__ __forceinline__ int32_t block_sum_i32(int32_t v, int32_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// A thread handles groups of 16 codes: group g covers k in [16g, 16g+16).
// Loads of one batch (kBatch groups per thread, 4 x 8 bytes each) are all
// issued before any is used; addresses past the row end are clamped and the
// values replaced by zeros (K % 4 == 0, so 4-value pieces never straddle).
constexpr int kBatch = 4;
constexpr int kOneBatchK = 16 * kBatch * kThreads;  // rows up to this stay in registers

struct Group {
  uint2 v[4];
};

__device__ __forceinline__ void load_group(const uint16_t* __restrict__ xr, int k, int g,
                                           Group& o) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 16 * g + 4 * j;
    const uint2 v = *reinterpret_cast<const uint2*>(xr + min(e, k - 4));
    o.v[j] = (e < k) ? v : make_uint2(0u, 0u);
  }
}

__device__ __forceinline__ uint32_t group_absmax(const Group& G) {
  uint32_t a = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) a = max(a, absmax_bits4(G.v[j].x, G.v[j].y));
  return a;
}

__device__ __forceinline__ void quant_group(const Group& G, float s, int32_t (&q)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    q[4 * j + 0] = quant_i8(bf16_to_f32(G.v[j].x & 0xFFFFu), s);
    q[4 * j + 1] = quant_i8(bf16_to_f32(G.v[j].x >> 16), s);
    q[4 * j + 2] = quant_i8(bf16_to_f32(G.v[j].y & 0xFFFFu), s);
    q[4 * j + 3] = quant_i8(bf16_to_f32(G.v[j].y >> 16), s);
  }
}

// Quantizes one bf16 row of length k; `emit(g, codes)` stores group g for
// every g < ngroups (groups past the row end carry zero codes).
template <typename Emit>
__device__ __forceinline__ float quant_row(const uint16_t* __restrict__ xr, int k, int ngroups,
                                           uint32_t* red, Emit emit) {
  const int tid = threadIdx.x;
  if (ngroups * 16 <= kOneBatchK) {
    Group G[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) load_group(xr, k, tid + kThreads * b, G[b]);
    uint32_t a = 0;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) a = max(a, group_absmax(G[b]));
    const float s = act_scale(bf16_to_f32(block_max_u32(a, red)));
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int g = tid + kThreads * b;
      if (g < ngroups) {
        int32_t q[16];
        quant_group(G[b], s, q);
        emit(g, q);
      }
    }
    return s;
  }
  uint32_t a = 0;
  for (int g0 = 0; g0 < ngroups; g0 += kThreads * kBatch) {
    Group G[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) load_group(xr, k, g0 + tid + kThreads * b, G[b]);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) a = max(a, group_absmax(G[b]));
  }
  const float s = act_scale(bf16_to_f32(block_max_u32(a, red)));
  for (int g0 = 0; g0 < ngroups; g0 += kThreads * kBatch) {
    Group G[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) load_group(xr, k, g0 + tid + kThreads * b, G[b]);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int g = g0 + tid + kThreads * b;
      if (g < ngroups) {
        int32_t q[16];
        quant_group(G[b], s, q);
        emit(g, q);
      }
    }
  }
  return s;
}

__device__ __forceinline__ void load16_codes(const int8_t* __restrict__ qr, int k, int k0,
                                             int32_t (&q)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t v = (k0 + 4 * j < k) ? *reinterpret_cast<const uint32_t*>(qr + k0 + 4 * j) : 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) q[4 * j + b] = (int32_t)(int8_t)(v >> (8 * b));
  }
}

// Internal layout of 16 codes: dword a, byte b = code 4b + a.
__device__ __forceinline__ v4i transpose16(const int32_t (&q)[16]) {
  v4i o;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    uint32_t d = ((uint32_t)q[a] & 0xFFu) | (((uint32_t)q[4 + a] & 0xFFu) << 8) |
                 (((uint32_t)q[8 + a] & 0xFFu) << 16) | (((uint32_t)q[12 + a] & 0xFFu) << 24);
    o[a] = (int32_t)d;
  }
  return o;
}

// Inspection output: codes 16g .. 16g+15 of a row of k codes in the natural
// layout, from dwords nat[j] holding codes 4j .. 4j+3 (byte i = code 4j + i).
// k % 4 == 0, so a dword never straddles the row end.
__device__ __forceinline__ void put_natural(int8_t* __restrict__ row, int k, int g,
                                            const uint32_t (&nat)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (16 * g + 4 * j < k) *reinterpret_cast<uint32_t*>(row + 16 * g + 4 * j) = nat[j];
}

// Stores the 16 codes of group g of a row (dword a, byte b = code 4b + a).
// GEMM order: the group's 16 bytes as they are.  Decode order: within each
// 32-code block (groups 2i, 2i+1), dwords 0 and 2 of group 2i, dwords 0 and
// 2 of group 2i+1, then dwords 1 and 3 of each -- the order in which the
// decode kernel's paired matrix-core ops take them.
__device__ __forceinline__ void put_group(v4i* __restrict__ qv, int g, v4i v, bool paired) {
  if (!paired) {
    qv[g] = v;
    return;
  }
  typedef int32_t v2i __attribute__((ext_vector_type(2)));
  int8_t* blk = reinterpret_cast<int8_t*>(qv) + 32 * (g >> 1) + 8 * (g & 1);
  *reinterpret_cast<v2i*>(blk) = v2i{v.x, v.z};
  *reinterpret_cast<v2i*>(blk + 16) = v2i{v.y, v.w};
}

__global__ __launch_bounds__(kThreads) void act_quant_public_kernel(
    const uint16_t* __restrict__ x, int k, int8_t* __restrict__ q, float* __restrict__ x_scale) {
  __shared__ uint32_t red[4];
  const int64_t m = blockIdx.x;
  int8_t* qr = q + m * k;
  const float s = quant_row(x + m * k, k, (k + 15) / 16, red, [&](int g, const int32_t(&c)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (16 * g + 4 * j < k) {
        uint32_t d = ((uint32_t)c[4 * j] & 0xFFu) | (((uint32_t)c[4 * j + 1] & 0xFFu) << 8) |
                     (((uint32_t)c[4 * j + 2] & 0xFFu) << 16) |
                     (((uint32_t)c[4 * j + 3] & 0xFFu) << 24);
        *reinterpret_cast<uint32_t*>(qr + 16 * g + 4 * j) = d;
      }
    }
  });
  if (threadIdx.x == 0) x_scale[m] = s;
}

// Wave-wide max / sum by DPP steps (quad swaps, row rotations) and four
// readlanes; every lane active.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad 1032
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad 2301
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}

// Rows with k % 8 == 0 (16-byte aligned): thread t owns the 16-code groups
// t + kThreads * b, two 16-byte loads each, all issued before any is used.
// The codes are packed straight into the internal order with the unsigned
// byte conversion (q + 128 is an exact integer in [0, 255]) and one xor per
// dword; the code sum comes from byte sums.  One barrier for the absmax, one
// for the code sum.
__device__ __forceinline__ void quant_row_internal_fast(const uint16_t* __restrict__ xr, int k,
                                                        int ngroups, v4i* __restrict__ qv,
                                                        uint32_t* red, int32_t* qsum,
                                                        float* x_scale, bool paired,
                                                        int8_t* nat_row, float* ins_xs,
                                                        int32_t* ins_qs) {
  constexpr int NB = kBatch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  v4i lo[NB], hi[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int g = tid + kThreads * b;
    const int e0 = min(16 * g, k - 8), e1 = min(16 * g + 8, k - 8);
    lo[b] = *reinterpret_cast<const v4i*>(xr + e0);
    hi[b] = *reinterpret_cast<const v4i*>(xr + e1);
    if (16 * g >= k) lo[b] = v4i{0, 0, 0, 0};
    if (16 * g + 8 >= k) hi[b] = v4i{0, 0, 0, 0};
  }
  uint32_t amax = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    amax = max(amax, max(max(absmax_bits4((uint32_t)lo[b].x, (uint32_t)lo[b].y),
                             absmax_bits4((uint32_t)lo[b].z, (uint32_t)lo[b].w)),
                         max(absmax_bits4((uint32_t)hi[b].x, (uint32_t)hi[b].y),
                             absmax_bits4((uint32_t)hi[b].z, (uint32_t)hi[b].w))));
  amax = wave_reduce(amax, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  const float s = act_scale(bf16_to_f32(max(max(red[0], red[1]), max(red[2], red[3]))));
  uint32_t usum = 0;  // sum of q + 128 over this thread's groups
  int ng = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int g = tid + kThreads * b;
    if (g < ngroups) {
      const uint32_t w[8] = {(uint32_t)lo[b].x, (uint32_t)lo[b].y, (uint32_t)lo[b].z,
                             (uint32_t)lo[b].w, (uint32_t)hi[b].x, (uint32_t)hi[b].y,
                             (uint32_t)hi[b].z, (uint32_t)hi[b].w};
      uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
        float t = __uint_as_float(bits) * s;
        t = fminf(fmaxf(rintf(t), -128.0f), 127.0f) + 128.0f;
        d[e & 3] = __builtin_amdgcn_cvt_pk_u8_f32(t, (uint32_t)(e >> 2), d[e & 3]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) usum = __builtin_amdgcn_sad_u8(d[a], 0u, usum);
      ++ng;
      if (nat_row) {  // inspection: byte i of natural dword j = byte j of d[i]
        uint32_t nat[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t v = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) v |= ((d[i] >> (8 * j)) & 0xFFu) << (8 * i);
          nat[j] = v ^ 0x80808080u;
        }
        put_natural(nat_row, k, g, nat);
      }
      put_group(qv, g,
                v4i{(int32_t)(d[0] ^ 0x80808080u), (int32_t)(d[1] ^ 0x80808080u),
                    (int32_t)(d[2] ^ 0x80808080u), (int32_t)(d[3] ^ 0x80808080u)},
                paired);
    }
  }
  int32_t sum = (int32_t)usum - 128 * 16 * ng;
  sum = (int32_t)wave_reduce((uint32_t)sum, [](uint32_t x, uint32_t y) { return x + y; });
  __syncthreads();  // red[] is reused
  if (lane == 0) red[wave] = (uint32_t)sum;
  __syncthreads();
  if (tid == 0) {
    const int32_t total = (int32_t)(red[0] + red[1] + red[2] + red[3]);
    *qsum = total;
    *x_scale = s;
    if (ins_qs) *ins_qs = total;
    if (ins_xs) *ins_xs = s;
  }
}

// Rows of bf16 input with k % 8 == 0, in the GEMM's order: a row of up to
// 256 groups of 16 codes has one wave, a row of up to 512 or 1024 groups two
// or four (`J.wpr`), so that one instance of four groups per lane covers
// every row at full occupancy.  Lane l of a row's wave w owns groups
// l + 64 (w + wpr b), b < 4, two 16-byte loads each, all issued before any is
// used.  Absmax and code sum are wave reductions, and a row's waves combine
// theirs through LDS: one barrier each, taken by the whole workgroup (all of
// a block's rows belong to one job, so wpr is the same for every wave of
// it).  q = rint(x * s) with |x * s| <= 127 * (1 + 2^-24) (s = RN(127 /
// amax)), so the clamp to [-128, 127] never binds; adding 1.5 * 2^23 to
// t = RN(x * s) rounds to an integer with ties to even and leaves q in two's
// complement in the low byte of the sum's bits, which byte permutes gather
// into the internal order (dword a, byte b = code 4b + a).
constexpr int kRowsNBW = 4;  // groups per lane

// The job of block b in one round trip to the kernel-argument segment: lane
// j (of each 16) reads job j's first block (row_begin) and descriptor, a
// ballot picks the job that holds b, and its words are broadcast with
// readlane (`first`: the job's row_begin entry).  (Looking up
// the job's index first and then its descriptor is two dependent round trips
// before the first activation load: 3B-class layer at M = 16 18.93 -> 18.44
// us per step, 8B-class layer at M = 8 19.5 -> 18.9 us.  A single job needs
// no lookup and reads its descriptor directly.)
static_assert(sizeof(ActQuantJob) % 16 == 0, "a job descriptor is read as 16-byte words");
__device__ __forceinline__ ActQuantJob select_job(int count, int b, int* first = nullptr) {
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const ActQuantArgs* ka = reinterpret_cast<const ActQuantArgs*>(kp);
  const int j = threadIdx.x & 15;
  constexpr int kWords = sizeof(ActQuantJob) / 16;
  v4i words[kWords];
  const v4i* src = reinterpret_cast<const v4i*>(&ka->j[j]);
#pragma unroll
  for (int i = 0; i < kWords; ++i) words[i] = src[i];
  const int beg = ka->row_begin[j];
  const int nxt = ka->row_begin[j < kMaxProj - 1 ? j + 1 : j];
  __builtin_amdgcn_sched_barrier(0);
  const int end = (j + 1 < count) ? nxt : 0x7FFFFFFF;
  const unsigned long long hit = __ballot(j < count && b >= beg && b < end);
  const int pi = __builtin_ctzll(hit) & 15;
  ActQuantJob J;
  int32_t* dst = reinterpret_cast<int32_t*>(&J);
#pragma unroll
  for (int i = 0; i < kWords; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[4 * i + c] = __builtin_amdgcn_readlane(words[i][c], pi);
  if (first) *first = __builtin_amdgcn_readlane(beg, pi);
  return J;
}

// INS: some job has inspection outputs (a separate instance, so that the
// bench path carries none of their registers).
template <bool INS>
__global__ __launch_bounds__(kThreads) void act_quant_rows_kernel(const ActQuantArgs a) {
  constexpr int NBW = kRowsNBW;
  __shared__ uint32_t red[2][kThreads / 64];
  const int b = blockIdx.x;
  if (b >= a.zero_blocks_begin) {
    const int64_t nzb = (int64_t)(gridDim.x - a.zero_blocks_begin);
    for (int64_t i = (int64_t)(b - a.zero_blocks_begin) * kThreads + threadIdx.x; i < a.zero_words;
         i += nzb * kThreads)
      a.zero[i] = 0;
    return;
  }
  // a.row_begin holds each job's first block here
  int first = 0;
  const ActQuantJob J = a.count > 1 ? select_job(a.count, b, &first) : a.j[0];
  const int lw = J.wpr == 1 ? 0 : (J.wpr == 2 ? 1 : 2);  // log2 of the waves per row
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int sub = wave & ((1 << lw) - 1);  // this wave's part of the row
  const int m = ((b - first) << (2 - lw)) + (wave >> lw);
  if (lw == 0 && m >= J.m_pad) return;  // past the job's rows (no barrier follows)
  const bool data = m < J.m;            // else a padding row (or past the rows): zero codes
  const int k = J.k, ngroups = J.ldq / 16;
  const int kg = k >> 4;  // groups holding data (a last half group: k % 16 == 8)
  const uint16_t* xr = J.x + (int64_t)(data ? m : 0) * k;
  v4i lo[NBW], hi[NBW];
#pragma unroll
  for (int bb = 0; bb < NBW; ++bb) {
    const int g = lane + 64 * (sub + (bb << lw));
    lo[bb] = hi[bb] = v4i{0, 0, 0, 0};
    if (data && 16 * g < k) {
      lo[bb] = *reinterpret_cast<const v4i*>(xr + 16 * g);
      if (16 * g + 8 < k) hi[bb] = *reinterpret_cast<const v4i*>(xr + 16 * g + 8);
    }
  }
  uint32_t amax = 0;
#pragma unroll
  for (int bb = 0; bb < NBW; ++bb)
    amax = max(amax, max(max(absmax_bits4((uint32_t)lo[bb].x, (uint32_t)lo[bb].y),
                             absmax_bits4((uint32_t)lo[bb].z, (uint32_t)lo[bb].w)),
                         max(absmax_bits4((uint32_t)hi[bb].x, (uint32_t)hi[bb].y),
                             absmax_bits4((uint32_t)hi[bb].z, (uint32_t)hi[bb].w))));
  amax = wave_reduce(amax, [](uint32_t x, uint32_t y) { return max(x, y); });
  const int w0 = wave & ~((1 << lw) - 1);  // the row's first wave
  if (lw > 0) {
    if (lane == 0) red[0][wave] = amax;
    __syncthreads();
    amax = max(red[0][w0], red[0][w0 + 1]);
    if (lw == 2) amax = max(amax, max(red[0][w0 + 2], red[0][w0 + 3]));
  }
  const float s = act_scale(bf16_to_f32(amax));
  const bool active = m < J.m_pad;
  v4i* qv = reinterpret_cast<v4i*>(J.q + (int64_t)(active ? m : 0) * J.ldq);
  int8_t* nat_row = (INS && data && J.ins_q) ? J.ins_q + (int64_t)m * k : nullptr;
  int32_t sum = 0;
#pragma unroll
  for (int bb = 0; bb < NBW; ++bb) {
    const int g = lane + 64 * (sub + (bb << lw));
    if (!active || g >= ngroups) continue;
    if (!data || g > kg || (g == kg && 16 * g >= k)) {  // padding: zero codes
      qv[g] = v4i{0, 0, 0, 0};
      continue;
    }
    const uint32_t w[8] = {(uint32_t)lo[bb].x, (uint32_t)lo[bb].y, (uint32_t)lo[bb].z,
                           (uint32_t)lo[bb].w, (uint32_t)hi[bb].x, (uint32_t)hi[bb].y,
                           (uint32_t)hi[bb].z, (uint32_t)hi[bb].w};
    uint32_t r[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
      r[e] = __float_as_uint(__uint_as_float(bits) * s + 12582912.0f);
    }
    v4i o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t l2 = __builtin_amdgcn_perm(r[q + 4], r[q], 0x0c0c0400u);
      const uint32_t h2 = __builtin_amdgcn_perm(r[q + 12], r[q + 8], 0x0c0c0400u);
      o[q] = (int32_t)__builtin_amdgcn_perm(h2, l2, 0x05040100u);
      sum = __builtin_amdgcn_sdot4(o[q], 0x01010101, sum, false);
    }
    qv[g] = o;
    if (INS && nat_row) {  // inspection: natural dword j, byte i = byte j of o[i]
      uint32_t nat[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sel = 0x0c0c0000u | ((4u + j) << 8) | (uint32_t)j;
        const uint32_t l2 = __builtin_amdgcn_perm((uint32_t)o[1], (uint32_t)o[0], sel);
        const uint32_t h2 = __builtin_amdgcn_perm((uint32_t)o[3], (uint32_t)o[2], sel);
        nat[j] = __builtin_amdgcn_perm(h2, l2, 0x05040100u);
      }
      put_natural(nat_row, k, g, nat);
    }
  }
  sum = (int32_t)wave_reduce((uint32_t)sum, [](uint32_t x, uint32_t y) { return x + y; });
  if (lw > 0) {
    if (lane == 0) red[1][wave] = (uint32_t)sum;
    __syncthreads();
    sum = (int32_t)(red[1][w0] + red[1][w0 + 1]);
    if (lw == 2) sum += (int32_t)(red[1][w0 + 2] + red[1][w0 + 3]);
  }
  if (data && sub == 0 && lane == 0) {
    J.qsum[m] = sum;
    J.x_scale[m] = s;
    if (INS && J.ins_qs) J.ins_qs[m] = sum;
    if (INS && J.ins_xs) J.ins_xs[m] = s;
  }
}

__global__ __launch_bounds__(kThreads) void act_quant_internal_kernel(const ActQuantArgs a) {
  __shared__ uint32_t red[4];
  const int b = blockIdx.x;
  if (b >= a.zero_blocks_begin) {
    const int64_t nzb = (int64_t)(gridDim.x - a.zero_blocks_begin);
    for (int64_t i = (int64_t)(b - a.zero_blocks_begin) * kThreads + threadIdx.x; i < a.zero_words;
         i += nzb * kThreads)
      a.zero[i] = 0;
    return;
  }
  const ActQuantJob J = a.count > 1 ? select_job(a.count, b) : a.j[0];
  const int m = b - J.row_begin;
  int8_t* qr = J.q + (int64_t)m * J.ldq;
  if (m >= J.m) {  // padding row: zero codes
    for (int g = threadIdx.x; g < J.ldq / 16; g += kThreads)
      reinterpret_cast<v4i*>(qr)[g] = v4i{0, 0, 0, 0};
    return;
  }
  int32_t sum = 0;
  v4i* qv = reinterpret_cast<v4i*>(qr);
  float s = 0.0f;
  int8_t* nat_row = (J.x && J.ins_q) ? J.ins_q + (int64_t)m * J.k : nullptr;
  if (J.x && (J.k & 7) == 0 && J.ldq / 16 <= kThreads * kBatch) {
    quant_row_internal_fast(J.x + (int64_t)m * J.k, J.k, J.ldq / 16, qv, red, J.qsum + m,
                            J.x_scale + m, J.paired != 0, nat_row,
                            J.ins_xs ? J.ins_xs + m : nullptr, J.ins_qs ? J.ins_qs + m : nullptr);
    return;
  }
  if (J.x) {
    s = quant_row(J.x + (int64_t)m * J.k, J.k, J.ldq / 16, red,
                  [&](int g, const int32_t(&c)[16]) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) sum += c[i];
                    put_group(qv, g, transpose16(c), J.paired != 0);
                    if (nat_row) {
                      uint32_t nat[4];
#pragma unroll
                      for (int j = 0; j < 4; ++j)
                        nat[j] = ((uint32_t)c[4 * j] & 0xFFu) |
                                 (((uint32_t)c[4 * j + 1] & 0xFFu) << 8) |
                                 (((uint32_t)c[4 * j + 2] & 0xFFu) << 16) |
                                 (((uint32_t)c[4 * j + 3] & 0xFFu) << 24);
                      put_natural(nat_row, J.k, g, nat);
                    }
                  });
  } else {
    const int8_t* qin = J.q_in + (int64_t)m * J.k;
    for (int g = threadIdx.x; g < J.ldq / 16; g += kThreads) {
      int32_t c[16];
      load16_codes(qin, J.k, 16 * g, c);
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += c[i];
      put_group(qv, g, transpose16(c), J.paired != 0);
    }
  }
  sum = block_sum_i32(sum, reinterpret_cast<int32_t*>(red));
  if (threadIdx.x == 0) {
    J.qsum[m] = sum;
    if (J.x) J.x_scale[m] = s;
    if (J.x && J.ins_qs) J.ins_qs[m] = sum;
    if (J.x && J.ins_xs) J.ins_xs[m] = s;
  }
}

}  // namespace

hipError_t launch_act_quant_public(const uint16_t* x, int64_t m, int64_t k, int8_t* q,
                                   float* x_scale, hipStream_t s) {
  act_quant_public_kernel<<<(unsigned)m, kThreads, 0, s>>>(x, (int)k, q, x_scale);
  return hipGetLastError();
}

hipError_t launch_act_quant_internal(const ActQuantArgs& a, int total_rows, hipStream_t s) {
  ActQuantArgs args = a;
  int zero_blocks = 0;
  if (args.zero_words > 0) {
    int64_t per = (int64_t)kThreads * 16;
    int64_t zb = (args.zero_words + per - 1) / per;
    zero_blocks = (int)(zb > 1024 ? 1024 : zb);
  }
  // one to four waves per row when every job is bf16 input in the GEMM's
  // code order with 16-byte rows of at most 16384 codes, at any row count
  // (mid-M layers of 119-896 rows: 0.25-0.3 us faster than a workgroup per
  // row).  The decode kernel's paired order keeps a workgroup per row:
  // written in that order by this kernel, the 2048 x 2048 projection at
  // M = 8 took 9.90 against 9.46 us.
  bool rows_ok = args.count > 0;
  for (int i = 0; i < args.count; ++i) {
    const ActQuantJob& J = args.j[i];
    rows_ok = rows_ok && J.x != nullptr && (J.k & 7) == 0 && !J.paired &&
              J.ldq / 16 <= 64 * kRowsNBW * 4;
  }
  if (rows_ok) {
    // blocks of 4 / wpr rows; a.row_begin becomes each job's first block
    int blocks = 0;
    for (int i = 0; i < args.count; ++i) {
      ActQuantJob& J = args.j[i];
      const int g = J.ldq / 16;
      J.wpr = g <= 64 * kRowsNBW ? 1 : (g <= 2 * 64 * kRowsNBW ? 2 : 4);
      args.row_begin[i] = blocks;
      blocks += (J.m_pad * J.wpr + kThreads / 64 - 1) / (kThreads / 64);
    }
    args.zero_blocks_begin = blocks;
    const dim3 grid((unsigned)(blocks + zero_blocks));
    bool ins = false;
    for (int i = 0; i < args.count; ++i)
      ins = ins || args.j[i].ins_q || args.j[i].ins_xs || args.j[i].ins_qs;
    if (ins)
      act_quant_rows_kernel<true><<<grid, kThreads, 0, s>>>(args);
    else
      act_quant_rows_kernel<false><<<grid, kThreads, 0, s>>>(args);
    return hipGetLastError();
  }
  args.zero_blocks_begin = total_rows;
  act_quant_internal_kernel<<<(unsigned)(total_rows + zero_blocks), kThreads, 0, s>>>(args);
  return hipGetLastError();
}

}  // namespace bl
