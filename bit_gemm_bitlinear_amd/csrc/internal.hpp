// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

constexpr int kMaxProj = 16;

// Decode path (M <= 16) limits.
constexpr int kDecodeMaxM = 16;
constexpr int kDecodeMaxTww = 4;      // 16-row tiles per wave
// 52 KB: 16 token rows of 3072 codes (plus row padding) fit, so the 3B-class
// layer's 3072-wide projections need no K split across workgroups at M = 16
// (measured: 26.6 -> 23.4 us per layer); a multiple of 4 KB, so the code
// staging of 256 threads covers it in whole 16-byte units.
#ifndef BL_DECODE_LDS_A
#define BL_DECODE_LDS_A (52 * 1024)
#endif
constexpr int kDecodeLdsA = BL_DECODE_LDS_A;  // LDS for a workgroup's activation codes
static_assert(kDecodeLdsA % (16 * 256) == 0, "staging units of 256 threads cover the budget");

// Activation codes for the contraction kernels are kept in an internal
// layout: rows padded to a multiple of 256 codes (zero filled), and inside
// every group of 16 codes the 4x4 byte transpose described in common.hpp.
// For the decode kernel the four dwords of each group are further placed in
// the order its paired matrix-core ops read (see put_group in act_quant.hip).
constexpr int kKPad = 256;

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---- activation quantization (act_quant.hip) ----
struct ActQuantJob {
  const uint16_t* x;   // [m][k] bf16 (nullptr: take codes from q_in)
  const int8_t* q_in;  // [m][k] int8 natural layout (used when x == nullptr)
  int8_t* q;           // [m_pad][ldq] internal layout (written)
  float* x_scale;      // [m] (written when x != nullptr)
  int32_t* qsum;       // [m] row sums of the codes (written)
  int32_t k, ldq, m, m_pad;
  int32_t row_begin;   // first block of this job in the launch
  int32_t paired;      // 1: the decode kernel's order (put_group in act_quant.hip), 0: the GEMM's
};

struct ActQuantArgs {
  ActQuantJob j[kMaxProj];
  int32_t count;
  int32_t zero_blocks_begin;  // blocks from here on only zero `zero`
  int32_t* zero;              // region cleared by the same launch (split-K partials)
  int64_t zero_words;         // its size in int32 words
};

hipError_t launch_act_quant_internal(const ActQuantArgs& a, int total_rows, hipStream_t s);
hipError_t launch_act_quant_public(const uint16_t* x, int64_t m, int64_t k, int8_t* q,
                                   float* x_scale, hipStream_t s);

// ---- decode contraction (decode.hip) ----
// Fused activation quantization inside the decode kernel: each workgroup
// reads the whole bf16 rows (at most kFusedMaxElems values, 16-byte chunks
// held in registers) and quantizes them itself.
constexpr int kFusedMaxM = 4;
constexpr int kFusedChunks = 8;  // 16-byte chunks of x per thread
constexpr int64_t kFusedMaxElems = (int64_t)kFusedChunks * 8 * 256;

struct DecodeProj {
  const uint8_t* packed;
  const float* w_scale;
  uint16_t* y;         // bf16 output, or nullptr
  int32_t* acc_out;    // int32 output when y == nullptr
  const uint16_t* x;   // fused: bf16 activations [m][k]; nullptr otherwise
  const int8_t* q;     // not fused: internal-layout codes [m][ldq]
  const float* x_scale;
  const int32_t* qsum;
  int32_t* part;       // [m][n] int32 split-K partials (zeroed beforehand)
  uint32_t* count;     // [ngroups] split-K arrival counters (zeroed beforehand)
  int32_t n, k, ldq;
  int32_t wk;          // waves sharing one row tile along K (1, 2 or 4)
  int32_t tww;         // 16-row tiles per wave
  int32_t kspw;        // K slabs (256 codes) per WG
  int32_t ksplit;      // WGs sharing one row group along K
  int32_t tiled;       // 1: weights in the 16-row tiled layout (common.hpp)
};

struct DecodeArgs {
  int32_t wg_begin[kMaxProj];  // first WG of each projection
  DecodeProj p[kMaxProj];
  int32_t count;
  int32_t m;
  int32_t load_mode;  // 0: 16-byte rows, 1: 4-byte rows, 2: byte rows
  int32_t lds_row;    // LDS row stride of the staged codes (bytes)
};

struct DecodePlan {
  int32_t wk, tww, kspw, ksplit, ngroups;
  bool fused;
};
DecodePlan plan_decode(int64_t m, int64_t n, int64_t k, int mode);
bool plan_decode_split(int64_t m, int32_t count, const int64_t* ns, const int64_t* ks, int mode,
                       int cus, DecodePlan* plans);
int device_cu_count();  // compute units of the current device (cached per device)
size_t decode_lds_bytes(int64_t m, int lds_row);
hipError_t launch_decode(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s);

// ---- prefill contraction (prefill.hip) ----
constexpr int kPrefillBM = 128;  // token rows per tile
#ifndef BL_PREFILL_BN
#define BL_PREFILL_BN 256
#endif
constexpr int kPrefillBN = BL_PREFILL_BN;  // output columns per tile, 16-byte aligned weight rows
constexpr int kPrefillNarrowBN = 128;  // the same, narrow tiles (the last round of a launch)
constexpr int kPrefillRegBN = 256;  // output columns per tile, other weight rows
inline int prefill_bn(int load_mode) { return load_mode == 0 ? kPrefillBN : kPrefillRegBN; }
#ifndef BL_PREFILL_WGS_PER_CU
#define BL_PREFILL_WGS_PER_CU 2
#endif
// Workgroups of the main prefill kernel that the LDS and registers allow per CU.
constexpr int kPrefillWgsPerCu = BL_PREFILL_WGS_PER_CU;

struct PrefillProj {
  const uint8_t* packed;
  const float* w_scale;
  uint16_t* y;
  int32_t* acc_out;
  const int8_t* q;      // internal layout [m_pad][ldq]
  const float* x_scale;
  const int32_t* qsum;
  int32_t n, k, ldq;    // n: output columns of this entry
  int32_t tiles_n;      // ceil(n / tile width)
  int32_t ldy;          // output row stride (elements of y or acc_out)
  int32_t narrow;       // 1: tiles of kPrefillNarrowBN columns (main variant only)
  // K split across workgroups (main variant only): part kp of a tile covers
  // slabs [kp * kspw, (kp + 1) * kspw) and writes its int32 sums to
  // part[kp][m][n] (row stride n); prefill_finish_kernel adds the parts.
  int32_t ksplit, kspw;
  int32_t* part;
  int32_t tiled;        // 1: weights in the 16-row tiled layout (common.hpp)
};

struct PrefillArgs {
  int32_t tile_begin[kMaxProj];  // first tile of each projection in the launch
  int32_t fin_begin[kMaxProj];   // first 8-output piece of each projection (finish)
  PrefillProj p[kMaxProj];
  int32_t count;
  int32_t m;
  int32_t tiles_m;
  int32_t load_mode;
};

// MI355X workgroup slots for the K-split plan of the prefill launch (256 CUs,
// two workgroups each): fixed, so that workspace sizes depend on shapes only.
constexpr int kPrefillPlanSlots = 512;
constexpr int kPrefillSlab = 128;  // codes per K slab of the main variant
// Slabs (128 codes) per K part: at least this many, and the plan splits a
// projection only when its K is over twice the launch's average load per slot.
constexpr int kPrefillMinPartSlabs = 16;
constexpr int kPrefillMaxSplit = 16;

hipError_t launch_prefill(const PrefillArgs& a, int total_tiles, hipStream_t s);
// Adds the K parts of the split projections and writes their outputs.
hipError_t launch_prefill_finish(const PrefillArgs& a, int total_pieces, hipStream_t s);

// ---- weight preparation (pack.hip) ----
hipError_t launch_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* w_scale,
                       unsigned long long* buckets, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* u, hipStream_t s);
// Row-major packed weights <-> the 16-row tiled layout (n % 16 == 0,
// k % 256 == 0); `untile` runs the inverse permutation.
hipError_t launch_tile(const uint8_t* src, int64_t n, int64_t k, uint8_t* dst, bool untile,
                       hipStream_t s);

}  // namespace bl
