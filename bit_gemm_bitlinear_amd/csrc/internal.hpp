// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

constexpr int kMaxProj = 16;
constexpr int kMaxDevices = 64;  // device indices the per-device caches cover

int current_device_index();  // hipGetDevice, clamped to [0, kMaxDevices)

// Decode path (M <= 16) limits.
constexpr int kDecodeMaxM = 16;
constexpr int kDecodeMaxTww = 4;      // 16-row tiles per wave (per-projection plans)
// 16-byte weight chunks a streaming wave targets in the per-projection
// plans.  Layers whose staged-code plans (5-16 token rows) keep at least one
// workgroup per CU at the larger target take it: each workgroup then streams
// more weight bytes per staged code byte.  Measured on the 8B-class layer:
// 21.9 -> 19.2 us at M = 5, 22.4 -> 19.5 us at M = 8, 30.3 -> 27.9 us at
// M = 16.  (The 3B-class layer at M = 16 would drop to 156 workgroups on 256
// CUs at 48 chunks, and took 22.7 against 19.3 us.)
constexpr int kDecodeWaveChunks = 24;
constexpr int kDecodeWaveChunksStaged = 32;
constexpr int kDecodeRedTww = 7;      // the same, any plan (sizes the in-LDS partial sums)
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
  int32_t row_begin;   // first block (or row) of this job in the launch
  int32_t paired;      // 1: the decode kernel's order (put_group in act_quant.hip), 0: the GEMM's
  int32_t wpr;         // waves per row of the wave-per-row kernel (set at its launch)
  // optional inspection outputs (bf16 input only; nullptr: not written): the
  // codes in the natural layout [m][k], the scales [m] and the code sums [m]
  int8_t* ins_q;
  float* ins_xs;
  int32_t* ins_qs;
};

struct ActQuantArgs {
  ActQuantJob j[kMaxProj];
  int32_t count;
  int32_t zero_blocks_begin;  // blocks from here on only zero `zero`
  int32_t* zero;              // region cleared by the same launch (split-K partials)
  int64_t zero_words;         // its size in int32 words
  // the jobs' row_begin again, as one contiguous array: a workgroup finds its
  // job with one argument load instead of one per job
  int32_t row_begin[kMaxProj];
};

hipError_t launch_act_quant_internal(const ActQuantArgs& a, int total_rows, hipStream_t s);
hipError_t launch_act_quant_public(const uint16_t* x, int64_t m, int64_t k, int8_t* q,
                                   float* x_scale, hipStream_t s);

// ---- decode contraction (decode.hip, decode_fused.hip, decode_kernels.hpp) ----
// Fused activation quantization inside the decode kernel: each workgroup
// reads the whole bf16 rows of up to kFusedMaxM tokens (16-byte chunks held
// in registers, at most fused_max_elems values) and quantizes them itself.
// (Measured with 8 rows: a 2048 x 2048 projection at M = 8 took 10.4 us
// fused against 9.8 us with the separate quantization launch, so 5-8 rows
// stage codes prepared by act_quant.hip.)
constexpr int kFusedMaxM = 4;
constexpr int kFusedChunks1 = 8;   // 16-byte chunks of x per thread, one token row
constexpr int kFusedChunksN = 24;  // the same, 2 to 4 token rows
// 2 to 4 rows whose codes exceed kFusedChunksN per thread, in the split
// shape only (its activation waves hold no weight ring): 4 rows of 14336, the
// 8B-class layer's down projection at M = 4.  A kernel instance of its own
// (kFusedBigSlots row slots), so that the other fused launches keep the
// shorter loops.
constexpr int kFusedChunksSplit = 28;
constexpr int kFusedBigSlots = 5;
inline int64_t fused_max_elems(int64_t m, bool split = false) {
  return (int64_t)(m == 1 ? kFusedChunks1 : (split ? kFusedChunksSplit : kFusedChunksN)) * 8 * 256;
}
// Code rows of a workgroup in the layer-level split plan (one workgroup per
// CU, so more LDS than the per-projection plans' kDecodeLdsA): 4 rows of
// 14336 codes fit.
constexpr int kDecodeSplitLdsA = 60 * 1024;
// Row slots of the kernel instance that fuses the quantization of m rows.
inline int fused_rows(int64_t m) { return m == 1 ? 1 : 4; }

struct DecodeProj {
  const uint8_t* packed;
  const float* w_scale;
  uint16_t* y;         // bf16 output, or nullptr
  int32_t* acc_out;    // int32 accumulators [m][n] (as well as y when both are set), or nullptr
  const uint16_t* x;   // fused: bf16 activations [m][k]; nullptr otherwise
  // Not fused: the staged inputs -- internal-layout codes [m][ldq], scales
  // and code sums prepared by act_quant.hip.  Fused: optional inspection
  // outputs the kernel writes (codes in the natural layout [m][k], scales,
  // code sums), or nullptr.
  int8_t* q;
  float* x_scale;
  int32_t* qsum;
  int32_t n, k, ldq;
  int32_t wk;          // waves sharing one row tile along K (1, 2 or 4)
  int32_t tww;         // 16-row tiles per wave
  int32_t kspw;        // K slabs (256 codes) per WG
  int32_t ksplit;      // WGs sharing one row group along K
  int32_t tiled;       // 1: weights in the 16-row tiled layout (common.hpp)
};
static_assert(sizeof(DecodeProj) == 96, "six 16-byte words");

// Fields of a projection that only the epilogue needs, kept apart from
// DecodeProj: every workgroup fetches its descriptor before its first load,
// and that fetch is shorter the fewer 16-byte words it has.
struct DecodeEpi {
  const uint16_t* bias;  // [n] bf16 added to y, or nullptr
  const uint16_t* res;   // [m][n] bf16 added to y after the bias (may be y itself), or nullptr
  int32_t* part;         // [m][n] int32 split-K partials (zeroed beforehand)
  uint32_t* count;       // [ngroups] split-K arrival counters (zeroed beforehand)
};

struct DecodeArgs {
  int32_t wg_begin[kMaxProj];  // first WG of each projection
  DecodeProj p[kMaxProj];
  DecodeEpi epi[kMaxProj];
  int32_t count;
  int32_t m;
  int32_t load_mode;  // 0: 16-byte rows, 1: 4-byte rows, 2: byte rows
  int32_t lds_row;    // LDS row stride of the staged codes (bytes)
  // The split shape's waves meet through LDS counters polled at most
  // wait_polls times (0: a wait gives up at once).  A workgroup whose wait
  // gave up writes NaN (bf16) or INT32_MIN (int32) outputs and, if status is
  // set, ORs 1 into *status.
  int32_t* status;
  int32_t wait_polls;
};
constexpr int32_t kDefaultWaitPolls = 1 << 24;

struct DecodePlan {
  int32_t wk, tww, kspw, ksplit, ngroups;
  bool fused;
};
DecodePlan plan_decode(int64_t m, int64_t n, int64_t k, int mode,
                       int target = kDecodeWaveChunks);
// have_x: the activations are bf16, so rows that fit may be quantized in the
// kernel (and may then use the larger LDS budget of the split plan).
bool plan_decode_split(int64_t m, int32_t count, const int64_t* ns, const int64_t* ks, int mode,
                       int cus, bool have_x, DecodePlan* plans);
int device_cu_count();  // compute units of the current device (cached per device)
size_t decode_lds_bytes(int64_t m, int lds_row);
hipError_t launch_decode(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s);
// The instances that fuse the quantization of 2 to 4 token rows.
hipError_t launch_decode_rows(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s,
                              bool epi, bool big);

// ---- prefill contraction (prefill.hip) ----
constexpr int kPrefillBM = 128;  // token rows per tile (register-staged variant; main variant's largest)
// Token rows per tile of the main variant: tiles of 32 or 64 rows for
// 16 < M <= 64 (the mid-M range, where 128-row tiles would mostly multiply
// padding rows), 128 otherwise.
// Token rows per tile of the main variant: 32 up to 32 rows, 64 up to 128
// rows, then 128.  Between 65 and 128 rows, two 64 x 256 tiles replace a
// 128 x 128 one (the launch then fills the slots with wide tiles): the same
// operations on 20% fewer operand bytes per tile.  Measured: 3B-class layer
// at M = 96 38.5 -> 35.2 us, M = 128 40.1 -> 36.0 us; the 8B-class layer
// lost 1.3-1.4 us at those sizes.  Up to 192 rows was mixed (3B-class M = 192
// +3.3 us, 8B-class -2.1 us), so larger M keeps 128-row tiles.
inline int prefill_bm(int64_t m, int load_mode) {
  if (load_mode != 0) return kPrefillBM;
  return m <= 32 ? 32 : (m <= 128 ? 64 : kPrefillBM);
}
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
  int32_t* acc_out;     // int32 accumulators (as well as y when both are set), or nullptr
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
  const uint16_t* bias; // [n] bf16 added to y (this entry's columns), or nullptr
  const uint16_t* res;  // [m][ldy] bf16 added to y after the bias (may be y), or nullptr
};

struct PrefillArgs {
  int32_t tile_begin[kMaxProj];  // first tile of each projection in the launch
  int32_t fin_begin[kMaxProj];   // first 8-output piece of each projection (finish)
  PrefillProj p[kMaxProj];
  int32_t count;
  int32_t m;
  int32_t tiles_m;
  int32_t load_mode;
  int32_t bm;  // token rows per tile (prefill_bm)
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
// bf16 u / w_scale [n][k] from packed weights in either layout.
hipError_t launch_export_bf16(const uint8_t* packed, int64_t n, int64_t k, bool tiled,
                              const float* w_scale, uint16_t* out, hipStream_t s);
// Row-major packed weights <-> the 16-row tiled layout (n % 16 == 0,
// k % 256 == 0); `untile` runs the inverse permutation.
hipError_t launch_tile(const uint8_t* src, int64_t n, int64_t k, uint8_t* dst, bool untile,
                       hipStream_t s);

}  // namespace bl
