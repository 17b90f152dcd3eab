// Device helpers shared by the BitLinear kernels (gfx950).
//
// Formulas follow the Falcon-Edge blog ("A series of powerful, universal and
// fine-tunable 1.58-bit language models", section "Falcon-Edge, a series of
// universal models"): activation_norm_quant, _weight_quant and
// BitLinear.post_quant_process.  All float arithmetic is single IEEE fp32
// operations with round-to-nearest-even (no contraction into FMAs, correctly
// rounded division), so results are bit-identical to a plain fp32 evaluation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Every product and sum is rounded on its own (the quantization and
// division steps depend on it), whatever contraction the build would allow.
#pragma clang fp contract(off)

namespace bl {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

// Address-space casts.  Pointers rebuilt from broadcast lane values lose the
// compiler's knowledge that they point to global memory, which would turn
// every access into a flat access (slower, and counted by both the vector
// and the scalar/LDS memory counters).  G() marks global memory, C() marks
// read-only data that may be read with scalar loads.
#define BL_GLOBAL __attribute__((address_space(1)))
#define BL_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ BL_GLOBAL T* G(T* p) {
  return (BL_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ const BL_CONST T* C(const T* p) {
  return (const BL_CONST T*)p;
}

// A uniform fp32 value read through the vector-memory path (a raw buffer
// load of 4 bytes).  It retires on the vector-memory counter, in order with
// the loads issued around it; an ordinary uniform load becomes a scalar load,
// which retires on the counter that LDS operations share, so every LDS or
// cross-lane wait after it would also wait for that memory round trip.
__device__ __forceinline__ float load_f32_vmem(const float* p) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, 4, 0x00020000);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// fp32(1e-5): the lower clamp of the absmax / absmean denominators.
constexpr float kEps = 1e-5f;

// The 16-row tiled weight layout (N % 16 == 0, K % 256 == 0).  The same
// bytes as the row-major [N][K/4] packing, permuted inside each block of 16
// rows: the block keeps its 16 * K/4 bytes in place, as 1 KB tiles of 16 rows
// x 64 packed bytes (256 weights) taken along K, and inside a tile the
// 16-byte chunk g (0..3) of row r (0..15) sits at 256 g + 16 r.  One tile is
// then exactly what 64 lanes read for one 16-row operand of the 16x16x64
// matrix-core op (lane 16 g + r: row r, chunk g), as one contiguous 1 KB.
// Byte offset of the 16-byte chunk at row byte `o` (a multiple of 16) of
// weight row `row`:
__host__ __device__ __forceinline__ int64_t tiled_chunk_offset(int64_t row, int64_t o,
                                                               int64_t rowbytes) {
  return (row >> 4) * 16 * rowbytes + 1024 * (o >> 6) + 256 * ((o >> 4) & 3) + 16 * (row & 15);
}

// 2-bit codes of 16 packed weights -> 4 dwords of int8 codes (0..3).
// Byte b of the packed dword holds weights 4b..4b+3 (2 bits each, least
// significant first).  Output dword a, byte b, holds the code of weight
// 4b + a: a 4x4 transpose of the natural order that costs one shift and
// one mask per dword.  Activations are stored in the same transposed order
// (see act_quant.hip), so the pairing of codes with activations is exact.
__device__ __forceinline__ v4i decode16(uint32_t p) {
  v4i r;
  r.x = (int32_t)(p & 0x03030303u);
  r.y = (int32_t)((p >> 2) & 0x03030303u);
  r.z = (int32_t)((p >> 4) & 0x03030303u);
  r.w = (int32_t)((p >> 6) & 0x03030303u);
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Per-token scale from the row's absmax: 127 / max(amax, 1e-5).
__device__ __forceinline__ float act_scale(float amax) {
  return 127.0f / fmaxf(amax, kEps);
}

// One int8 code: clamp(round_half_even(x * s), -128, 127).
__device__ __forceinline__ int32_t quant_i8(float x, float s) {
  float t = rintf(x * s);
  t = fminf(fmaxf(t, -128.0f), 127.0f);
  return (int32_t)t;
}

// One ternary code c = u + 1 with u = clamp(round_half_even(w * s), -1, 1).
__device__ __forceinline__ uint32_t ternary_code(float w, float s) {
  float t = rintf(w * s);
  t = fminf(fmaxf(t, -1.0f), 1.0f);
  return (uint32_t)(int32_t)(t + 1.0f);
}

// Output: bf16(acc / (x_scale * w_scale)), one fp32 product, one division.
__device__ __forceinline__ uint16_t dequant_bf16(int32_t acc, float xs, float ws) {
  float d = xs * ws;
  float yf = (float)acc / d;
  return f32_to_bf16(yf);
}

}  // namespace bl

#include "row_div.hpp"

namespace bl {

// Same result as dequant_bf16 for a row whose divisor was prepared once.
__device__ __forceinline__ uint16_t dequant_bf16_row(int32_t acc, const RowDiv& r) {
  return f32_to_bf16(row_div((float)acc, r));
}

// The same when the divisor is known to be in the range of the fast step
// (row_div_setup's `fast`), without the per-value check.
__device__ __forceinline__ uint16_t dequant_bf16_fast(int32_t acc, float d, float y) {
  return f32_to_bf16(row_div_fast((float)acc, d, y));
}

// Two outputs converted together (one v_cvt_pk_bf16_f32): lo in bits 0-15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

// bf16 a + b the way a bf16 tensor add rounds (the bias line of
// BitLinear.forward): both widened to fp32, one fp32 add, the sum rounded to
// bf16 (round to nearest even).
__device__ __forceinline__ uint16_t add_bf16(uint16_t a, uint16_t b) {
  return f32_to_bf16(bf16_to_f32(a) + bf16_to_f32(b));
}

// The same for two pairs held in dwords (bf16 in bits 0-15 and 16-31).
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  return pack_bf16x2(bf16_to_f32(a & 0xFFFFu) + bf16_to_f32(b & 0xFFFFu),
                     __uint_as_float(a & 0xFFFF0000u) + __uint_as_float(b & 0xFFFF0000u));
}

// Largest magnitude pattern of four bf16 values held in two dwords; the
// bit pattern of |x| orders like |x| for finite values.
__device__ __forceinline__ uint32_t absmax_bits4(uint32_t lo, uint32_t hi) {
  uint32_t a = max(lo & 0x7FFFu, (lo >> 16) & 0x7FFFu);
  uint32_t b = max(hi & 0x7FFFu, (hi >> 16) & 0x7FFFu);
  return max(a, b);
}

__device__ __forceinline__ v4i mfma_16x16x64_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace bl
