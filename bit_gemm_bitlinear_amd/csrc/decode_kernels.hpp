// Decode contraction (M <= 16 tokens): acc[m][n] = sum_k q[m][k] * u[n][k],
// then y = bf16(acc / (x_scale[m] * w_scale)) -- the F.linear call and
// post_quant_process of BitLinear.forward in the Falcon-Edge blog ("A series
// of powerful, universal and fine-tunable 1.58-bit language models", section
// "Falcon-Edge, a series of universal models"), in exact integer arithmetic.
//
// This is bound by HBM bandwidth on the packed weights (2 bits per weight),
// so the kernel is organised around streaming them once:
//  * work unit: a workgroup owns 16*TW consecutive weight rows per group of
//    streaming waves and a range of K (all of it unless K is split for LDS
//    space).  Split shape (one workgroup per CU): waves 0-3 stream through a
//    16-deep load ring per lane while waves 4-7 prepare the activation codes;
//    ring shape (several workgroups per CU): four waves prepare the codes,
//    then stream through an 8-deep ring;
//  * activations: for small M*K the workgroup quantizes the bf16 rows itself
//    (activation_norm_quant: exact integer absmax over the bf16 magnitude
//    bits, one fp32 division, one multiply and one rounding add per code)
//    straight into LDS -- no separate launch; otherwise it stages codes
//    prepared by act_quant.hip.  Either way the activation loads reach the
//    memory pipeline before the weight loads (a barrier orders them in the
//    split shape): behind a full weight stream they would arrive microseconds
//    later;
//  * each 16 packed bytes hold 64 weights = four K-steps of one row for the
//    16x16x64 int8 matrix-core op; they are expanded in registers with five
//    bit operations per packed dword (mma_chunk), and sum q*u = sum q*c - sum q
//    restores the ternary weights u = c - 1 from the codes c;
//  * token rows m >= M of the 16-row A operand repeat row 0 (rows of the
//    product do not mix; output rows m >= M are never stored);
//  * the streaming waves may split K, and their partial sums meet in LDS.
// Loads past the end of a row or past the last row are clamped to valid
// addresses instead of masked: the activation codes there are zero (rows of
// codes are zero-padded) and output columns of rows >= N are never stored.
#pragma once

#include "common.hpp"
#include "internal.hpp"

#include <atomic>
#include <type_traits>

namespace bl {

namespace {

#ifndef BL_DECODE_WINDOW
#define BL_DECODE_WINDOW 8
#endif
static_assert(BL_DECODE_WINDOW % 4 == 0, "ring slots hold whole tile rounds");

constexpr int kWindow = BL_DECODE_WINDOW;  // 16-byte weight chunks in flight per lane
constexpr int kWaveChunks = kDecodeWaveChunks;  // target chunks streamed per wave (ring shape)
constexpr int kWaveMaxChunks = 24;              // most chunks per wave at that target
constexpr int kWaveMaxChunksStaged = kDecodeWaveChunksStaged;  // staged-code instances
constexpr int kSplitRing = 16;             // load ring per lane of the split shape
constexpr int kStageUnits = kDecodeLdsA / 16 / 256;  // 16-byte code units per activation thread

// 16 bytes of a packed row at byte offset `off` (a multiple of 16).  Parts
// past `rowbytes` read the row's last bytes instead (multiplied by zero).
// MODE 0: rowbytes % 16 == 0 (one 128-bit load); 1: rowbytes % 4 == 0;
// 2: any length.  A compile-time choice keeps the loads branch-free.
template <int MODE>
__device__ __forceinline__ v4i load_w16(const uint8_t* __restrict__ row, int off, int rowbytes) {
  v4i r;
  if constexpr (MODE == 0) {
    r = __builtin_nontemporal_load(G(reinterpret_cast<const v4i*>(row + min(off, rowbytes - 16))));
  } else if constexpr (MODE == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = __builtin_nontemporal_load(
          G(reinterpret_cast<const int32_t*>(row + min(off + 4 * j, rowbytes - 4))));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t d = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        d |= (uint32_t)__builtin_nontemporal_load(G(row + min(off + 4 * j + b, rowbytes - 1)))
             << (8 * b);
      r[j] = (int32_t)d;
    }
  }
  return r;
}

// The workgroup's projection, found in one round trip to the kernel-argument
// segment: lane j (of each 16) reads projection j's first WG index and
// descriptor, a ballot picks the projection containing this WG, and its
// descriptor words are broadcast with readlane.  (Indexing the argument
// struct by a computed projection index would cost a second, dependent
// round trip before any weight load could be issued.)
__device__ __forceinline__ DecodeProj select_proj(int count, int* wl, int* proj) {
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const DecodeArgs* ka = reinterpret_cast<const DecodeArgs*>(kp);
  const int j = threadIdx.x & 15;
  const int beg = ka->wg_begin[j];
  const int nxt = ka->wg_begin[j < kMaxProj - 1 ? j + 1 : j];
  constexpr int kWords = sizeof(DecodeProj) / 16;
  static_assert(sizeof(DecodeProj) % 16 == 0, "descriptor is read as 16-byte words");
  v4i words[kWords];
  const v4i* src = reinterpret_cast<const v4i*>(&ka->p[j]);
#pragma unroll
  for (int i = 0; i < kWords; ++i) words[i] = src[i];
  __builtin_amdgcn_sched_barrier(0);
  const int end = (j + 1 < count) ? nxt : 0x7FFFFFFF;
  const int b = (int)blockIdx.x;
  const unsigned long long hit = __ballot(j < count && b >= beg && b < end);
  const int pi = __builtin_ctzll(hit) & 15;
  DecodeProj P;
  int32_t* dst = reinterpret_cast<int32_t*>(&P);
#pragma unroll
  for (int i = 0; i < kWords; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[4 * i + c] = __builtin_amdgcn_readlane(words[i][c], pi);
  *wl = b - __builtin_amdgcn_readlane(beg, pi);
  *proj = pi;
  return P;
}

// Wave-wide max / sum: four DPP steps reduce each row of 16 lanes (quad
// swaps, then rotations by 4 and 8), and the four row results are combined
// from lanes 0, 16, 32 and 48.  Needs every lane active.  (Shuffles through
// ds_bpermute would put six dependent LDS round trips on the path.)
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

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return max(x, y); });
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
  return (int32_t)wave_reduce((uint32_t)v, [](uint32_t x, uint32_t y) { return x + y; });
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1 (a compile-time loop).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

// Per-WG scalars shared by the activation side and the epilogue.
struct Shared {
  RowDiv rd[kDecodeMaxM];        // per-row divisors x_scale * w_scale
  int32_t qs[kDecodeMaxM];       // code sums
  uint32_t part[4][kFusedMaxM];  // per-wave absmax of each token row
  int32_t flag;
  // split shape: LDS handshakes between the two wave roles
  int32_t amax_count;  // activation waves that posted their absmax
  int32_t ready;       // activation waves done with codes and scalars
  int32_t bad;         // an activation wave's wait gave up
};

// Waits until *c reaches `target` (other waves of this workgroup add to it).
// Only LDS is involved, so a waiting wave's outstanding weight loads are left
// alone.  The waves of a workgroup are resident together, so the counter does
// get there; the bound (`polls`) only guarantees an exit.  Returns false if
// the wait gave up: the caller then reports it and poisons its outputs rather
// than pass off what LDS held as a result.
__device__ __forceinline__ bool lds_wait(const int32_t* c, int target, int polls) {
  bool ok = false;
  for (int it = 0; it < polls; ++it) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return ok;
}

// Records a wait that gave up: once per wave, in the caller's status word.
__device__ __forceinline__ void report_giveup(const DecodeArgs& A) {
  if (A.status && (threadIdx.x & 63) == 0) atomicOr(A.status, 1);
}

// Workgroup barrier ordering LDS only: weight loads in flight are not waited
// for (a full __syncthreads fence could wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Publishes this wave's LDS writes, then adds one to *c.
__device__ __forceinline__ void lds_post(int32_t* c) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Writes one output: bf16, or the int32 accumulator (forward_acc).  With EPI
// (a separate kernel instance for the extra epilogue work) the bf16 output
// gets the bias and then the residual added (BitLinear.forward's bias line,
// each add rounded to bf16), and int32 accumulators are written next to it
// where both are asked for (inspection).  A workgroup whose wait gave up
// (`bad`) writes NaN / INT32_MIN.
template <bool EPI>
__device__ __forceinline__ void store_out(const DecodeProj& P, const DecodeEpi& E, int m, int n,
                                          int32_t acc, const Shared& sh, bool bad) {
  const int64_t o = (int64_t)m * P.n + n;
  if (P.y) {
    uint16_t v = bad ? (uint16_t)0x7FC0u : dequant_bf16_row(acc - sh.qs[m], sh.rd[m]);
    if constexpr (EPI) {
      if (E.bias) v = add_bf16(v, *G(E.bias + n));
      if (E.res) v = add_bf16(v, *G(E.res + o));
    }
    *G(P.y + o) = v;
  }
  if ((EPI || !P.y) && P.acc_out) *G(P.acc_out + o) = bad ? (int32_t)0x80000000u : acc - sh.qs[m];
}

// Stores the 16 codes of group g (dword a, byte b = code 4b + a of the group)
// into a row of the LDS code image.  Within each 32-code block (groups 2i,
// 2i+1 = halves h) the dwords are ordered for the paired matrix-core ops of
// mma_chunk: [a=0 of h=0, a=2 of h=0, a=0 of h=1, a=2 of h=1, a=1 of h=0,
// a=3 of h=0, a=1 of h=1, a=3 of h=1].
__device__ __forceinline__ void put_group(int8_t* row, int g, v4i v) {
  int8_t* blk = row + 32 * (g >> 1) + 8 * (g & 1);
  typedef int32_t v2i __attribute__((ext_vector_type(2)));
  *reinterpret_cast<v2i*>(blk) = v2i{v.x, v.z};
  *reinterpret_cast<v2i*>(blk + 16) = v2i{v.y, v.w};
}

// The activation side is run by 256 threads (xt = 0..255, four waves).
// load_codes issues its loads: the bf16 rows (fused quantization) or the
// codes act_quant.hip prepared, and w_scale.  FR: 0 for staged codes, else
// the token-row slots of the fused quantizer (1, 4 or 8), one kernel instance
// per bucket so that one row does not pay for the loops over eight.
template <bool SPLIT, int FR>
constexpr int kXChunks =
    FR == 0 ? kStageUnits
            : (FR == 1 ? kFusedChunks1 : (FR == kFusedBigSlots ? kFusedChunksSplit : kFusedChunksN));

template <bool SPLIT, int FR>
__device__ __forceinline__ void load_codes(const DecodeArgs& A, const DecodeProj& P, int sb, int ns,
                                           v4i (&xin)[kXChunks<SPLIT, FR>], float& ws) {
  constexpr bool FUSED = FR > 0;
  constexpr int NA = 256;
  constexpr int NX = kXChunks<SPLIT, FR>;
  const int M = A.m;
  const int xt = threadIdx.x & (NA - 1);
  if constexpr (FUSED) {
    // thread xt owns the 16-element groups xt + NA * i: two 16-byte chunks
    // each (rows are contiguous, k % 16 == 0)
    const int units = M * (P.k >> 4);
#pragma unroll
    for (int i = 0; i < NX / 2; ++i) {
      if (xt + NA * i < units) {
        const v4i* src = reinterpret_cast<const v4i*>(P.x + 16 * (int64_t)(xt + NA * i));
        xin[2 * i] = *G(src);
        xin[2 * i + 1] = *G(src + 1);
      }
    }
  } else {
    const int units = M * ns * 16;  // 16-byte code units of the staged K range
    const int upr = ns * 16;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int u = min(xt + NA * i, units - 1);
      const int m = u / upr, c = u - m * upr;
      xin[i] = *G(reinterpret_cast<const v4i*>(P.q + (int64_t)m * P.ldq + sb * 256 + c * 16));
    }
  }
  // w_scale through the vector-memory path: a scalar load would retire on
  // the counter that LDS operations share, so the first cross-lane or LDS
  // wait below would wait for it as well.
  ws = P.y ? load_f32_vmem(P.w_scale) : 0.0f;
}

// prepare_codes puts the activation codes of the WG's K range in LDS, plus
// the per-row code sums and divisors.  Fused: quantize the bf16 rows
// (activation_norm_quant: exact integer absmax over the bf16 magnitude bits,
// one fp32 division per row, one multiply and round per code).  Otherwise:
// stage the loaded codes.  The four waves meet through barriers (single
// shape) or LDS counters (split shape, where the streaming waves must not
// wait with them).
// `inspect` (fused, the projection's first workgroup): also write the codes
// in the natural layout and the scales to P.q and P.x_scale when those are set.
template <bool SPLIT, int FR>
__device__ __forceinline__ void prepare_codes(const DecodeArgs& A, const DecodeProj& P, int ns,
                                              const v4i (&xin)[kXChunks<SPLIT, FR>], const float ws,
                                              int8_t* __restrict__ lds, Shared& sh, bool inspect) {
  constexpr bool FUSED = FR > 0;
  constexpr int NA = 256;  // activation threads
  constexpr int NX = kXChunks<SPLIT, FR>;
  const int M = A.m;
  const int xt = threadIdx.x & (NA - 1);
  const int lane = xt & 63, xw = xt >> 6;
  const int lrow = A.lds_row;
  const int S = (P.k + 255) >> 8;
  const int units = FUSED ? M * (P.k >> 4) : M * ns * 16;
  if constexpr (!FUSED) {
    if (xt < M) {
      sh.qs[xt] = *G(P.qsum + xt);
      if (P.y) sh.rd[xt] = row_div_setup(*G(P.x_scale + xt) * ws);
    }
    const int upr = ns * 16;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int u = xt + NA * i;
      if (u < units) {  // already in the decode order (act_quant.hip)
        const int m = u / upr, c = u - m * upr;
        *reinterpret_cast<v4i*>(lds + m * lrow + 16 * c) = xin[i];
      }
    }
  } else {
    // row of each group without a division (M <= FR)
    const int gpr = P.k >> 4;  // groups per row
    int grow[NX / 2];
#pragma unroll
    for (int i = 0; i < NX / 2; ++i) {
      const int g = xt + NA * i;
      int r = 0;
#pragma unroll
      for (int j = 1; j < FR; ++j) r += (g >= j * gpr);
      grow[i] = r;
    }
    // per-row absmax over the bf16 magnitude bits (exact)
    uint32_t mx[FR];
#pragma unroll
    for (int r = 0; r < FR; ++r) mx[r] = 0;
#pragma unroll
    for (int i = 0; i < NX / 2; ++i) {
      if (xt + NA * i < units) {
        const v4i lo = xin[2 * i], hi = xin[2 * i + 1];
        const uint32_t a = max(max(absmax_bits4((uint32_t)lo.x, (uint32_t)lo.y),
                                   absmax_bits4((uint32_t)lo.z, (uint32_t)lo.w)),
                               max(absmax_bits4((uint32_t)hi.x, (uint32_t)hi.y),
                                   absmax_bits4((uint32_t)hi.z, (uint32_t)hi.w)));
#pragma unroll
        for (int r = 0; r < FR; ++r) mx[r] = (grow[i] == r) ? max(mx[r], a) : mx[r];
      }
    }
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      if (r < M) {
        const uint32_t v = wave_max(mx[r]);
        if (lane == 0) sh.part[xw][r] = v;
      }
    }
    if (xt < M) sh.qs[xt] = 0;
    if constexpr (SPLIT) lds_post(&sh.amax_count);
    // zero the padding codes [k, 256*S) of every row meanwhile
    const int pad0 = P.k, padg = (S * 256 - P.k) / 16;  // k % 16 == 0
    for (int i = xt; i < M * padg; i += NA) {
      int m = 0;
#pragma unroll
      for (int j = 1; j < FR; ++j) m += (i >= j * padg);
      const int c = i - m * padg;
      put_group(lds + m * lrow, (pad0 >> 4) + c, v4i{0, 0, 0, 0});
    }
    if constexpr (SPLIT) {
      if (!lds_wait(&sh.amax_count, 4, A.wait_polls)) {
        sh.bad = 1;  // published with the codes (lds_post below)
        report_giveup(A);
      }
    } else {
      lds_barrier();
    }
    float s[FR];
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      s[r] = 0.0f;
      if (r < M) {
        const uint32_t a = max(max(sh.part[0][r], sh.part[1][r]), max(sh.part[2][r], sh.part[3][r]));
        s[r] = act_scale(bf16_to_f32(a));
      }
    }
    // quantize a group: q = rint(x * s).  |x * s| <= 127 * (1 + 2^-24)
    // (s = RN(127 / amax), |x| <= amax), so the clamp to [-128, 127] never
    // binds and q lies in [-127, 127].  Adding 1.5 * 2^23 to t = RN(x * s)
    // rounds it to an integer with ties to even (the spacing of floats there
    // is 1, and 1.5 * 2^23 is even) and leaves q in two's complement in the
    // low byte of the sum's bits.  Element 4b + a of the group goes to byte b
    // of dword a (the weight decode's order), gathered by byte permutes.
    int32_t sum[FR];
#pragma unroll
    for (int r = 0; r < FR; ++r) sum[r] = 0;
#pragma unroll
    for (int i = 0; i < NX / 2; ++i) {
      const int g = xt + NA * i;
      if (g < units) {
        const int m = grow[i];
        float sc = s[0];
#pragma unroll
        for (int r = 1; r < FR; ++r) sc = (m == r) ? s[r] : sc;
        const uint32_t w[8] = {(uint32_t)xin[2 * i].x, (uint32_t)xin[2 * i].y,
                               (uint32_t)xin[2 * i].z, (uint32_t)xin[2 * i].w,
                               (uint32_t)xin[2 * i + 1].x, (uint32_t)xin[2 * i + 1].y,
                               (uint32_t)xin[2 * i + 1].z, (uint32_t)xin[2 * i + 1].w};
        uint32_t r[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
          const float t = __uint_as_float(bits) * sc;
          r[e] = __float_as_uint(t + 12582912.0f);
        }
        uint32_t d[4];
        int32_t part = 0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t lo = __builtin_amdgcn_perm(r[a + 4], r[a], 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(r[a + 12], r[a + 8], 0x0c0c0400u);
          d[a] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          part = __builtin_amdgcn_sdot4((int32_t)d[a], 0x01010101, part, false);
        }
#pragma unroll
        for (int r2 = 0; r2 < FR; ++r2) sum[r2] += (m == r2) ? part : 0;
        const int k0 = 16 * (g - m * gpr);
        put_group(lds + m * lrow, k0 >> 4,
                  v4i{(int32_t)d[0], (int32_t)d[1], (int32_t)d[2], (int32_t)d[3]});
        if (inspect && P.q) {  // natural order: byte e of the group = code e
          v4i nat;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = __builtin_amdgcn_perm(r[4 * j + 1], r[4 * j], 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(r[4 * j + 3], r[4 * j + 2], 0x0c0c0400u);
            nat[j] = (int32_t)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
          *G(reinterpret_cast<v4i*>(P.q + (int64_t)m * P.k + k0)) = nat;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      if (r < M) {
        const int32_t v = wave_sum(sum[r]);
        if (lane == 0) atomicAdd(&sh.qs[r], v);  // zeroed before the absmax meeting
      }
      if (xt == r && r < M && P.y) sh.rd[r] = row_div_setup(s[r] * ws);
      if (xt == r && r < M && inspect && P.x_scale) *G(P.x_scale + r) = s[r];
    }
  }
  if constexpr (SPLIT)
    lds_post(&sh.ready);
  else
    lds_barrier();
}

// Consumes one 16-byte weight chunk (64 weights of one row, four K-steps of
// the 16x16x64 int8 matrix-core op), expanded in registers to codes
// c = u + 1 (common.hpp).
//
// Two matrix-core ops per pair of packed dwords p, p': one on the codes of
// weights 4b and 4b+2 of each byte b (p & 0x03030303 and (p >> 4) &
// 0x03030303), one on 4x the codes of weights 4b+1 and 4b+3 (the same masks
// shifted by 2, with no shift back).  That is five bit operations per packed
// dword instead of seven; the second accumulator holds four times its sum,
// which is divided out exactly at the end.  The activation codes are laid out
// in LDS to match (put_group).
__device__ __forceinline__ void mma_chunk(v4i& acc1, v4i& acc4, const v4i (&a)[4], const v4i b) {
  constexpr uint32_t M1 = 0x03030303u, M4 = 0x0C0C0C0Cu;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t p0 = (uint32_t)b[2 * h], p1 = (uint32_t)b[2 * h + 1];
    const uint32_t t0 = p0 >> 4, t1 = p1 >> 4;
    const v4i b1 = v4i{(int32_t)(p0 & M1), (int32_t)(t0 & M1), (int32_t)(p1 & M1), (int32_t)(t1 & M1)};
    const v4i b4 = v4i{(int32_t)(p0 & M4), (int32_t)(t0 & M4), (int32_t)(p1 & M4), (int32_t)(t1 & M4)};
    acc1 = mfma_16x16x64_i8(a[2 * h], b1, acc1);
    acc4 = mfma_16x16x64_i8(a[2 * h + 1], b4, acc4);
  }
}

// EARLY (ring shape, several token rows): the first weight loads go out
// before the code preparation instead of after it.
// EPI: the extra epilogue work (inspection outputs, bias, residual) is
// compiled in (a separate kernel instance).
template <int TWW, int MODE, int FR, bool SPLIT, bool EARLY, bool EPI>
__device__ __forceinline__ void decode_body(const DecodeArgs& A, const DecodeProj& P,
                                            const DecodeEpi& E, int wl, int8_t* __restrict__ lds,
                                            Shared& sh) {
  constexpr int NT = SPLIT ? 512 : 256;
  const int M = A.m;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const bool streamer = tid < 256;  // waves 0-3 stream weights and hold the sums
  const int sw = wave & 3;
  // WG -> (row group, K part); streaming wave -> (row wave wr, K wave wk_i).
  // wk is 1, 2 or 4: shifts and masks, no divisions ahead of the first loads.
  const int lwk = __builtin_ctz((unsigned)P.wk);
  const int group = P.ksplit == 1 ? wl : wl / P.ksplit, kpart = wl - group * P.ksplit;
  const int wr = sw >> lwk, wki = sw & (P.wk - 1);
  const int rows_wg = (TWW * 64) >> lwk;
  const int row0 = group * rows_wg + wr * TWW * 16;
  const int S = (P.k + 255) >> 8;
  const int sb = kpart * P.kspw;
  const int ns = min(S, sb + P.kspw) - sb;  // slabs of this WG
  const int nsw = (ns + P.wk - 1) >> lwk;   // slabs per wave
  const int ws0 = min(ns, wki * nsw);       // first slab of this wave (relative)
  const int nw = min(ns, ws0 + nsw) - ws0;  // slabs of this wave (may be 0)
  const int rowbytes = P.k >> 2;
  const int lrow = A.lds_row;
  constexpr bool FUSED = FR > 0;
  const bool inspect = EPI && FUSED && wl == 0;  // one workgroup writes the inspection outputs
  bool bad = false;                       // split shape: a wait of this wave gave up

  // weights: this wave streams its TWW row tiles over its K slabs, slab-major
  // so each A fragment feeds TWW tiles.  Every load is unconditional (past
  // the end it repeats the last chunk, a cache hit that is never used), so
  // the memory-counter waits are exact.  Lane (ln, lg) takes row ln of the
  // row tile, bytes 16 lg.. of the slab's 64: in the row-major layout 16 rows
  // x 64 bytes, in the tiled layout (common.hpp) one contiguous 1 KB at
  // 16 * lane of the tile.  Both are one address formula with per-lane
  // constants, so the layout costs no branch.
  const int NI = TWW * nw;
  const int last = max(NI - 1, 0);
  const bool tl = P.tiled != 0;
  const int row_add = tl ? 0 : ln;
  const int row_max = tl ? P.n - 16 : P.n - 1;  // tiled: n % 16 == 0
  const int slab_bytes = tl ? 1024 : 64;
  const int lane_off = tl ? 16 * lane : 16 * lg;
  const int lim = tl ? 16 * rowbytes : rowbytes;  // bytes the clamp keeps the load in
  auto wload = [&](int it) {
    const int c = min(it, last);
    const int ls = c / TWW, t = c - ls * TWW;
    const int row = min(row0 + 16 * t + row_add, row_max);
    return load_w16<MODE>(P.packed + (int64_t)row * rowbytes, (sb + ws0 + ls) * slab_bytes + lane_off,
                          lim);
  };
  // token rows m >= M of the A operand repeat row 0: output rows m >= M
  // are never stored, and rows do not mix in the product
  const int8_t* abase = lds + (ln < M ? ln : 0) * lrow + 64 * lg + ws0 * 256;
  auto afrag = [&](int ls, v4i (&a)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const v4i*>(abase + ls * 256 + 16 * j);
  };
  v4i acc[TWW], acc4[TWW];  // sums over weights 4b, 4b+2 and 4x those over 4b+1, 4b+3
#pragma unroll
  for (int t = 0; t < TWW; ++t) acc[t] = acc4[t] = v4i{0, 0, 0, 0};

  if constexpr (SPLIT) {
    // waves 4-7 prepare the codes; waves 0-3 put all of their weight loads
    // in flight and start on them as soon as the codes are ready.  The
    // activation loads are issued before the workgroup's first barrier,
    // the weight loads after it, so that the activations do not queue
    // behind the weights.
    if (!streamer) {
      v4i xin[kXChunks<true, FR>];
      float ws;
      load_codes<true, FR>(A, P, sb, ns, xin, ws);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");  // counters are zero
      prepare_codes<true, FR>(A, P, ns, xin, ws, lds, sh, inspect);
    } else {
      // a ring of NC chunks per lane: every slot is refilled with the chunk
      // NC ahead right after it is read, so NC loads stay in flight until
      // the last round (which refills nothing)
      constexpr int NC = TWW == 3 ? 24 : (TWW == 7 ? 14 : kSplitRing);
      static_assert(NC % TWW == 0, "a ring slot always holds the same row tile");
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");  // counters zeroed
      __builtin_amdgcn_s_barrier();
      v4i ring[NC];
#pragma unroll
      for (int d = 0; d < NC; ++d) ring[d] = wload(d);
      __builtin_amdgcn_sched_barrier(0);
      if (!lds_wait(&sh.ready, 4, A.wait_polls)) {
        bad = true;
        report_giveup(A);
      }
      // an activation wave's give-up, published with `ready` (wave-uniform)
      bad = __builtin_amdgcn_readfirstlane((bad || sh.bad) ? 1 : 0) != 0;
      v4i a[4];
      auto round = [&](int base, auto refill) {
        static_for<NC>([&](auto dc) {
          constexpr int d = decltype(dc)::value;
          constexpr int t = d % TWW;  // base is a multiple of NC, NC of TWW
          const v4i b = ring[d];
          if constexpr (decltype(refill)::value) ring[d] = wload(base + NC + d);
          if (base + d < NI) {
            if constexpr (t == 0) afrag((base + d) / TWW, a);
            mma_chunk(acc[t], acc4[t], a, b);
          }
        });
      };
      const int rounds = max((NI + NC - 1) / NC, 1);
      for (int r = 0; r + 1 < rounds; ++r) round(r * NC, std::true_type{});
      round((rounds - 1) * NC, std::false_type{});
    }
  } else {
    // all four waves prepare the codes, then stream through a ring of
    // kWindow chunks (one round consumes slots 0..W-1; with REFILL each slot
    // is reloaded one round ahead right after it is read; rounds are nested
    // so every executed path is straight-line code)
    // With several token rows (EARLY) the first W weight loads go out right
    // behind the activation loads, so the longer code preparation overlaps
    // them; with one row it is short, and the activation loads fare better
    // alone.
    constexpr int W = kWindow;
    static_assert(W % 4 == 0, "a ring slot always holds the same row tile");
    v4i ring[W];
    auto fill = [&]() {
#pragma unroll
      for (int d = 0; d < W; ++d) ring[d] = wload(d);
      __builtin_amdgcn_sched_barrier(0);
    };
    {
      v4i xin[kXChunks<false, FR>];
      float ws;
      load_codes<false, FR>(A, P, sb, ns, xin, ws);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (EARLY) fill();
      prepare_codes<false, FR>(A, P, ns, xin, ws, lds, sh, inspect);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!EARLY) fill();
    v4i a[4];
    auto round = [&](int base, auto refill) {
      static_for<W>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int t = d % TWW;  // base is a multiple of W, W of TWW
        const int it = base + d;
        const v4i b = ring[d];
        if constexpr (decltype(refill)::value) ring[d] = wload(it + W);
        if (it < NI) {
          if constexpr (t == 0) afrag(it / TWW, a);
          mma_chunk(acc[t], acc4[t], a, b);
        }
      });
    };
    using Yes = std::true_type;
    using No = std::false_type;
    // three rounds at most for the fused-quantization instances, four for
    // the staged-code ones (the larger chunk target of big layers); the
    // fused instances keep their shorter code (a loop over rounds instead
    // of this nesting made the 2-4-row instances slower: 3B-class layer at
    // M = 4 19.4 against 13.1 us)
    static_assert(kWaveMaxChunks <= 3 * W, "at most three rounds");
    static_assert(kWaveMaxChunksStaged <= 4 * W, "at most four rounds");
    if (NI <= W) {
      round(0, No{});
    } else {
      round(0, Yes{});
      if (NI <= 2 * W) {
        round(W, No{});
      } else {
        round(W, Yes{});
        if constexpr (FR == 0) {
          if (NI <= 3 * W) {
            round(2 * W, No{});
          } else {
            round(2 * W, Yes{});
            round(3 * W, No{});
          }
        } else {
          round(2 * W, No{});
        }
      }
    }
  }

#pragma unroll
  for (int t = 0; t < TWW; ++t) acc[t] += acc4[t] >> 2;  // exact: multiples of 4

  // inspection: the code sums of the fused quantization (final once the codes
  // are posted, which every streaming wave has waited for)
  if (EPI && FUSED && inspect && P.qsum && tid < M) *G(P.qsum + tid) = sh.qs[tid];

  // epilogue.  Streaming lane (ln, lg) holds rows m = 4*lg + r of output
  // column row0 + 16*t + ln.
  if (P.wk == 1 && P.ksplit == 1) {
    if (!streamer) return;
#pragma unroll
    for (int t = 0; t < TWW; ++t) {
      const int n = row0 + 16 * t + ln;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * lg + r;
        if (m < M && n < P.n) store_out<EPI>(P, E, m, n, acc[t][r], sh, bad);
      }
    }
    return;
  }
  // K split across the streaming waves of a row group: partial sums meet in
  // LDS (a region after the staged codes, so no barrier is needed before
  // writing), then every wave of the WG finishes.
  int32_t* red = reinterpret_cast<int32_t*>(lds + M * lrow);
  if (streamer) {
#pragma unroll
    for (int t = 0; t < TWW; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * lg + r;
        if (m < M) red[((sw * TWW + t) * M + m) * 16 + ln] = acc[t][r];
      }
    }
    if constexpr (SPLIT)
      if (bad) sh.bad = 1;
  }
  __syncthreads();
  if constexpr (SPLIT) bad = __builtin_amdgcn_readfirstlane(sh.bad) != 0;
  // output idx -> row m and local column nl; with TWW a power of two,
  // rows_wg and TWW * 16 are too and the split is shifts and masks (seven
  // tiles per wave divide by constants)
  constexpr bool kPow2 = (TWW & (TWW - 1)) == 0;
  const int lrw = 31 - __builtin_clz(rows_wg), ltw = 31 - __builtin_clz(TWW * 16);
  const int nout = kPow2 ? (M << lrw) : M * rows_wg;  // outputs of this WG
  auto split_idx = [&](int idx, int& m, int& nl) {
    if constexpr (kPow2) {
      m = idx >> lrw;
      nl = idx & (rows_wg - 1);
    } else {
      m = idx / rows_wg;
      nl = idx - m * rows_wg;
    }
  };
  for (int idx = tid; idx < nout; idx += NT) {
    int m, nl;
    split_idx(idx, m, nl);
    const int g = kPow2 ? nl >> ltw : nl / (TWW * 16);  // g = row wave
    const int t = kPow2 ? (nl >> 4) & (TWW - 1) : (nl >> 4) % TWW, c = nl & 15;
    const int n = group * rows_wg + nl;
    int32_t v = 0;
    for (int q = 0; q < P.wk; ++q) v += red[(((g * P.wk + q) * TWW + t) * M + m) * 16 + c];
    if (n >= P.n) continue;
    if (P.ksplit == 1)
      store_out<EPI>(P, E, m, n, v, sh, bad);
    else
      atomicAdd(E.part + (int64_t)m * P.n + n, v);
  }
  if (P.ksplit == 1) return;

  // K split across WGs (never with fused quantization): the last WG of the
  // row group finishes (integer addition, so the arrival order does not
  // matter).  The partial sums above are device-scope atomics; once every
  // thread has seen its own acknowledged (memory counter at zero) and the
  // workgroup has met, the counter increment is ordered after all of them,
  // and the last WG reads the sums back with atomics as well.  No cache
  // write-back fence is needed for data that only atomics touch.  (Plain
  // device-coherent stores into per-part slices, read back with coherent
  // loads, were measured slower than these atomics.)
  if constexpr (FUSED) return;  // fused quantization never splits K across WGs
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) sh.flag = (atomicAdd(E.count + group, 1u) == (uint32_t)(P.ksplit - 1));
  __syncthreads();
  if (!sh.flag) return;
  // read-backs four at a time, all four in flight together
  for (int base = tid; base < nout; base += 4 * NT) {
    int32_t vals[4];
    int outm[4], outn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = base + NT * i;
      int nl;
      split_idx(idx, outm[i], nl);
      outn[i] = group * rows_wg + nl;
      vals[i] = (idx < nout && outn[i] < P.n)
                    ? atomicAdd(E.part + (int64_t)outm[i] * P.n + outn[i], 0)
                    : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (base + NT * i < nout && outn[i] < P.n)
        store_out<EPI>(P, E, outm[i], outn[i], vals[i], sh, bad);
  }
}

template <int TWW, int MODE, bool SPLIT, bool EARLY, bool EPI, int FR>
__device__ __forceinline__ void decode_tw(const DecodeArgs& A, const DecodeProj& P,
                                          const DecodeEpi& E, int wl, int8_t* lds, Shared& sh) {
  if constexpr (MODE == 0 && FR > 0) {
    if (P.x) {
      decode_body<TWW, MODE, FR, SPLIT, EARLY, EPI>(A, P, E, wl, lds, sh);
      return;
    }
  }
  decode_body<TWW, MODE, 0, SPLIT, EARLY, EPI>(A, P, E, wl, lds, sh);
}

// SPLIT: 8 waves, for launches that fit on the chip in one wave of WGs (the
// activation work of a WG then overlaps its weight stream instead of
// preceding it); otherwise 4 waves, so that several WGs share a CU.
// FR: row slots of the fused quantizer (0: every projection stages codes).
template <int MODE, bool SPLIT, bool EARLY, bool EPI, int FR>
__global__ __launch_bounds__(SPLIT ? 512 : 256) void decode_kernel(const DecodeArgs A) {
  extern __shared__ __align__(16) int8_t lds[];
  __shared__ Shared sh;
  if constexpr (SPLIT) {
    if (threadIdx.x == 0) {
      sh.amax_count = 0;
      sh.ready = 0;
      sh.bad = 0;
    }
  }
  int wl, pi;
  const DecodeProj P = select_proj(A.count, &wl, &pi);
  // the epilogue's fields: read where they are used (bias and residual only
  // in the EPI instance, the split-K buffers only when K is split)
  const DecodeEpi& E = A.epi[pi];
  switch (P.tww) {
    case 1: decode_tw<1, MODE, SPLIT, EARLY, EPI, FR>(A, P, E, wl, lds, sh); break;
    case 2: decode_tw<2, MODE, SPLIT, EARLY, EPI, FR>(A, P, E, wl, lds, sh); break;
    case 3:  // split-shape plans only
      if constexpr (SPLIT) decode_tw<3, MODE, SPLIT, EARLY, EPI, FR>(A, P, E, wl, lds, sh);
      break;
    case 7:  // split-shape plans only
      if constexpr (SPLIT) decode_tw<7, MODE, SPLIT, EARLY, EPI, FR>(A, P, E, wl, lds, sh);
      break;
    default: decode_tw<4, MODE, SPLIT, EARLY, EPI, FR>(A, P, E, wl, lds, sh); break;
  }
}

// Lets kernel K use up to `bytes` of dynamic LDS (needed above 64 KB); once
// per instantiation and device.
template <auto Kern>
hipError_t allow_lds(size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  static std::atomic<bool> done[kMaxDevices];
  const int dev = current_device_index();
  if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)decode_lds_bytes(kDecodeMaxM, kDecodeLdsA / kDecodeMaxM + 16));
  if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
  return e;
}

// Launches the decode kernel instance for the launch shape, with EPI and FR
// fixed by the caller.  Row-major weights of other alignments (MODE 1, 2)
// never fuse the quantization.
template <bool EPI, int FR>
hipError_t launch_decode_as(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s) {
  const bool split = a.load_mode == 0 && total_wgs <= device_cu_count();
  const dim3 grid((unsigned)total_wgs);
  hipError_t e = hipSuccess;
  if (a.load_mode == 0) {
    if (split) {
      e = allow_lds<&decode_kernel<0, true, false, EPI, FR>>(lds_bytes);
      if (e == hipSuccess) decode_kernel<0, true, false, EPI, FR><<<grid, 512, lds_bytes, s>>>(a);
    } else if constexpr (FR == kFusedBigSlots) {
      return hipErrorInvalidValue;  // not reached: only split plans fuse that many codes
    } else if (a.m > 1) {
      e = allow_lds<&decode_kernel<0, false, true, EPI, FR>>(lds_bytes);
      if (e == hipSuccess) decode_kernel<0, false, true, EPI, FR><<<grid, 256, lds_bytes, s>>>(a);
    } else {
      e = allow_lds<&decode_kernel<0, false, false, EPI, FR>>(lds_bytes);
      if (e == hipSuccess) decode_kernel<0, false, false, EPI, FR><<<grid, 256, lds_bytes, s>>>(a);
    }
  } else if constexpr (FR == 0) {
    if (a.load_mode == 1) {
      e = allow_lds<&decode_kernel<1, false, false, EPI, 0>>(lds_bytes);
      if (e == hipSuccess) decode_kernel<1, false, false, EPI, 0><<<grid, 256, lds_bytes, s>>>(a);
    } else {
      e = allow_lds<&decode_kernel<2, false, false, EPI, 0>>(lds_bytes);
      if (e == hipSuccess) decode_kernel<2, false, false, EPI, 0><<<grid, 256, lds_bytes, s>>>(a);
    }
  } else {
    return hipErrorInvalidValue;  // not reached: the host plans no fusion for MODE 1, 2
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

}  // namespace bl
