// extern "C" entry points of libbitlinear.so (declared in include/bitlinear.h):
// host-side argument validation, workspace layout and kernel dispatch.  No
// entry point allocates, frees or synchronizes; every argument is checked
// before anything is enqueued.
#include "../../include/bitlinear.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "internal.hpp"
#include "prefill_plan.hpp"

using namespace bl;

namespace {

constexpr int64_t kMaxK = int64_t(1) << 22;
constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxM = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr size_t kPackWorkspace = 256 * sizeof(unsigned long long);

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bl_status check_ptr(const void* p) {
  if (!p) return BL_EINVAL;
  if (!aligned16(p)) return BL_EALIGN;
  return BL_OK;
}

bl_status check_shape(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || n < 1 || k < 1) return BL_ESHAPE;
  if (k % 4 != 0 || k > kMaxK || n > kMaxN || m > kMaxM) return BL_ESHAPE;
  if (m * k >= kMaxElems || n * (k / 4) >= kMaxElems || m * n >= kMaxElems) return BL_ESHAPE;
  return BL_OK;
}

int load_mode_for(int64_t k) { return (k % 64 == 0) ? 0 : (k % 16 == 0) ? 1 : 2; }

// The 16-row tiled weight layout needs whole 16-row blocks and whole 1 KB
// tiles (256 weights of each of 16 rows).
bl_status check_tiled_shape(int64_t n, int64_t k) {
  return (n % 16 == 0 && k % 256 == 0) ? BL_OK : BL_ESHAPE;
}

// Workspace layout of a forward call (shared by the size query and the call).
struct Layout {
  bool decode;
  int load_mode;
  int32_t m_pad;
  int32_t bm;          // prefill: token rows per tile
  bool all_narrow;     // prefill: every tile of the launch is a narrow one
  size_t q_off[kMaxProj], xs_off[kMaxProj], qs_off[kMaxProj];
  size_t part_off[kMaxProj], cnt_off[kMaxProj];
  DecodePlan plan[kMaxProj];
  // prefill (main variant): K parts per projection and their int32 partial sums
  int32_t pf_ksplit[kMaxProj], pf_kspw[kMaxProj];
  size_t pf_part_off[kMaxProj];
  size_t zero_off, zero_bytes;
  size_t total;
};

int load_mode_for(int32_t count, const int64_t* ks) {
  int mode = 0;
  for (int i = 0; i < count; ++i) mode = std::max(mode, load_mode_for(ks[i]));
  return mode;
}

// `have_x`: the activations are bf16 (not caller-supplied codes), so small
// decode projections may quantize inside the contraction kernel and need no
// workspace for codes.
void make_layout(int32_t count, const int64_t* ns, const int64_t* ks, int64_t m, bool have_x,
                 Layout& L) {
  L.decode = m <= kDecodeMaxM;
  L.load_mode = load_mode_for(count, ks);
  L.bm = prefill_bm(m, L.load_mode);
  L.m_pad = L.decode ? (int32_t)m : (int32_t)round_up(m, L.bm);
  // A launch whose wide tiles would leave most workgroup slots empty (the
  // mid-M range: few token tiles) runs every tile narrow, twice as many.
  L.all_narrow = false;
  if (!L.decode && L.load_mode == 0) {
    int64_t wide = 0;
    for (int i = 0; i < count; ++i)
      wide += (int64_t)(L.m_pad / L.bm) * ((ns[i] + kPrefillBN - 1) / kPrefillBN);
    L.all_narrow = 2 * wide < kPrefillPlanSlots;
  }
  // decode: a layer that one workgroup per CU can cover takes the split
  // plan; otherwise each projection is planned on its own
  const bool split =
      L.decode &&
      plan_decode_split(m, count, ns, ks, L.load_mode, device_cu_count(), have_x, L.plan);
  // per-projection plans of staged codes (5-16 rows) take the larger chunk
  // target when the layer then still has a workgroup for every CU
  int target = kDecodeWaveChunks;
  if (L.decode && !split && m > kFusedMaxM) {
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
      const DecodePlan q = plan_decode(m, ns[i], ks[i], L.load_mode, kDecodeWaveChunksStaged);
      wgs += (int64_t)q.ngroups * q.ksplit;
    }
    if (wgs >= device_cu_count()) target = kDecodeWaveChunksStaged;
  }
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    L.q_off[i] = L.xs_off[i] = L.qs_off[i] = 0;
    if (L.decode) {
      if (!split) L.plan[i] = plan_decode(m, ns[i], ks[i], L.load_mode, target);
      L.plan[i].fused = L.plan[i].fused && have_x;
      if (L.plan[i].fused) continue;
    }
    const int64_t ldq = round_up(ks[i], kKPad);
    L.q_off[i] = off;
    off = align256(off + (size_t)L.m_pad * (size_t)ldq);
    L.xs_off[i] = off;
    off = align256(off + sizeof(float) * (size_t)m);
    L.qs_off[i] = off;
    off = align256(off + sizeof(int32_t) * (size_t)m);
  }
  L.zero_off = off;
  for (int i = 0; i < count; ++i) {
    L.part_off[i] = L.cnt_off[i] = 0;
    if (!L.decode) continue;
    if (L.plan[i].ksplit > 1) {
      L.part_off[i] = off;
      off = align256(off + sizeof(int32_t) * (size_t)(m * ns[i]));
      L.cnt_off[i] = off;
      off = align256(off + sizeof(uint32_t) * (size_t)L.plan[i].ngroups);
    }
  }
  L.zero_bytes = off - L.zero_off;
  // prefill: split the K of projections whose tiles would outlast the rest of
  // the launch (a plan from the shapes alone, so the size queries agree)
  for (int i = 0; i < count; ++i) {
    L.pf_ksplit[i] = 1;
    L.pf_kspw[i] = (int32_t)((ks[i] + kPrefillSlab - 1) / kPrefillSlab);
    L.pf_part_off[i] = 0;
  }
  if (!L.decode && L.load_mode == 0) {
    int64_t slabs[kMaxProj], tiles[kMaxProj];
    for (int i = 0; i < count; ++i) {
      slabs[i] = L.pf_kspw[i];
      const int64_t bn = L.all_narrow ? kPrefillNarrowBN : kPrefillBN;
      tiles[i] = (int64_t)(L.m_pad / L.bm) * ((ns[i] + bn - 1) / bn);
    }
    plan_ksplit(count, slabs, tiles, kPrefillPlanSlots, kPrefillMinPartSlabs, kPrefillMaxSplit,
                L.pf_ksplit, L.pf_kspw);
    for (int i = 0; i < count; ++i) {
      if (L.pf_ksplit[i] == 1) continue;
      L.pf_part_off[i] = off;
      off = align256(off + sizeof(int32_t) * (size_t)L.pf_ksplit[i] * (size_t)m * (size_t)ns[i]);
    }
  }
  // the size does not depend on which plan the device's CU count picks:
  // room for the per-projection plans' split-K partials is always counted
  // (at the default chunk target, whose plans have the most row groups)
  size_t ring = L.zero_off;
  for (int i = 0; L.decode && i < count; ++i) {
    const DecodePlan p = plan_decode(m, ns[i], ks[i], L.load_mode);
    if (p.ksplit > 1)
      ring = align256(align256(ring + sizeof(int32_t) * (size_t)(m * ns[i])) +
                      sizeof(uint32_t) * (size_t)p.ngroups);
  }
  off = std::max(off, ring);
  L.total = off > 0 ? off : 256;
}

struct ProjIO {
  const uint16_t* x;
  const int8_t* q_in;
  const uint8_t* packed;
  const float* w_scale;
  uint16_t* y;
  int32_t* acc;   // int32 accumulators: the output of forward_acc, or inspection
  int64_t n, k;
  int32_t tiled;  // 1: packed is in the 16-row tiled layout
  // inspection of the activation quantization (bf16 input), or nullptr
  int8_t* ins_q;
  float* ins_xs;
  int32_t* ins_qs;
  const uint16_t* bias;  // [n] bf16, or nullptr
  const uint16_t* res;   // [m][n] bf16, or nullptr
};

// Diagnostics of a call: the decode kernel's wait bound and status word.
struct CallDiag {
  int32_t* status = nullptr;
  int32_t wait_polls = kDefaultWaitPolls;
};

bl_status run_forward(int32_t count, const ProjIO* io, int64_t m, void* workspace,
                      size_t ws_bytes, hipStream_t stream, const CallDiag& diag = CallDiag()) {
  int64_t ns[kMaxProj], ks[kMaxProj];
  for (int i = 0; i < count; ++i) {
    ns[i] = io[i].n;
    ks[i] = io[i].k;
  }
  // The documented requirement (the size queries) is the layout with a code
  // region for every projection; a call that quantizes inside the
  // contraction kernel uses less of it.
  Layout L;
  make_layout(count, ns, ks, m, false, L);
  if (!workspace) return BL_EWORKSPACE;
  if (!aligned16(workspace)) return BL_EALIGN;
  if (ws_bytes < L.total) return BL_EWORKSPACE;
  if (io[0].x != nullptr) make_layout(count, ns, ks, m, true, L);
  char* ws = static_cast<char*>(workspace);

  const int load_mode = L.load_mode;

  // 1. activation codes (+ scales, code sums) of the projections that do not
  //    quantize inside the contraction kernel, and clearing of split-K partials
  ActQuantArgs qa = {};
  int8_t* qptr[kMaxProj];
  float* xsptr[kMaxProj];
  int32_t* qsptr[kMaxProj];
  int rows = 0, jobs = 0;
  for (int i = 0; i < count; ++i) {
    qptr[i] = reinterpret_cast<int8_t*>(ws + L.q_off[i]);
    xsptr[i] = reinterpret_cast<float*>(ws + L.xs_off[i]);
    qsptr[i] = reinterpret_cast<int32_t*>(ws + L.qs_off[i]);
    if (L.decode && L.plan[i].fused) continue;
    ActQuantJob& J = qa.j[jobs++];
    J.x = io[i].x;
    J.q_in = io[i].q_in;
    J.q = qptr[i];
    J.x_scale = xsptr[i];
    J.qsum = qsptr[i];
    J.k = (int32_t)ks[i];
    J.ldq = (int32_t)round_up(ks[i], kKPad);
    J.m = (int32_t)m;
    J.m_pad = L.m_pad;
    J.row_begin = rows;
    qa.row_begin[jobs - 1] = rows;
    J.paired = L.decode ? 1 : 0;
    J.ins_q = io[i].ins_q;
    J.ins_xs = io[i].ins_xs;
    J.ins_qs = io[i].ins_qs;
    rows += L.m_pad;
  }
  qa.count = jobs;
  qa.zero = reinterpret_cast<int32_t*>(ws + L.zero_off);
  qa.zero_words = (int64_t)(L.zero_bytes / sizeof(int32_t));
  if (jobs > 0 || qa.zero_words > 0)
    if (launch_act_quant_internal(qa, rows, stream) != hipSuccess) return BL_EHIP;

  // 2. contraction + dequantization
  if (L.decode) {
    DecodeArgs da = {};
    da.count = count;
    da.m = (int32_t)m;
    da.load_mode = load_mode;
    da.status = diag.status;
    da.wait_polls = diag.wait_polls;
    int wgs = 0, lds_row = 0;
    // Launch order: workgroups that finish last start first.  Those of a K
    // split across workgroups end with a round of atomics and a read-back
    // (3B-class layer at M = 16: 21.4 -> 20.5 us with them first); the rest
    // by weight bytes per workgroup, largest first (the caller's order when
    // equal: putting the 3B-class layer's longer-row but smaller down
    // projection workgroups first cost 0.8 us at M = 1).
    int order[kMaxProj];
    for (int i = 0; i < count; ++i) order[i] = i;
    auto wg_bytes = [&](int i) {
      const DecodePlan& p = L.plan[i];
      return (int64_t)(4 / p.wk) * p.tww * 16 * p.kspw * 64;
    };
    std::stable_sort(order, order + count, [&](int a, int b) {
      const bool sa = L.plan[a].ksplit > 1, sb = L.plan[b].ksplit > 1;
      if (sa != sb) return sa;
      return wg_bytes(a) > wg_bytes(b);
    });
    for (int o = 0; o < count; ++o) {
      const int i = order[o];
      DecodeProj& P = da.p[o];
      const DecodePlan& pl = L.plan[i];
      P.packed = io[i].packed;
      P.w_scale = io[i].w_scale;
      P.y = io[i].y;
      P.acc_out = io[i].acc;
      P.x = pl.fused ? io[i].x : nullptr;
      // fused: the kernel quantizes, and these are its inspection outputs
      P.q = pl.fused ? io[i].ins_q : qptr[i];
      P.x_scale = pl.fused ? io[i].ins_xs : xsptr[i];
      P.qsum = pl.fused ? io[i].ins_qs : qsptr[i];
      da.epi[o].part = pl.ksplit > 1 ? reinterpret_cast<int32_t*>(ws + L.part_off[i]) : nullptr;
      da.epi[o].count = pl.ksplit > 1 ? reinterpret_cast<uint32_t*>(ws + L.cnt_off[i]) : nullptr;
      P.n = (int32_t)ns[i];
      P.k = (int32_t)ks[i];
      P.ldq = (int32_t)round_up(ks[i], kKPad);
      da.epi[o].bias = io[i].bias;
      da.epi[o].res = io[i].res;
      P.wk = pl.wk;
      P.tww = pl.tww;
      P.kspw = pl.kspw;
      P.ksplit = pl.ksplit;
      P.tiled = io[i].tiled;
      da.wg_begin[o] = wgs;
      wgs += pl.ngroups * pl.ksplit;
      lds_row = std::max(lds_row, pl.kspw * 256 + 16);
    }
    for (int i = count; i < kMaxProj; ++i) da.wg_begin[i] = wgs;
    da.lds_row = lds_row;
    const size_t lds = decode_lds_bytes(m, lds_row);
    if (launch_decode(da, wgs, lds, stream) != hipSuccess) return BL_EHIP;
  } else {
    PrefillArgs pa = {};
    pa.count = count;
    pa.m = (int32_t)m;
    pa.tiles_m = L.m_pad / L.bm;
    pa.load_mode = load_mode;
    pa.bm = L.bm;
    const int32_t bn = L.all_narrow ? kPrefillNarrowBN : prefill_bn(load_mode);
    // Longest K first: the dispatcher hands out workgroups in launch order,
    // so the costliest tiles start first and the short ones fill in.
    int order[kMaxProj];
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order, order + count,
                     [&](int a, int b) { return L.pf_kspw[a] > L.pf_kspw[b]; });  // slabs per tile
    for (int o = 0; o < count; ++o) {
      const int i = order[o];
      PrefillProj& P = pa.p[o];
      P.packed = io[i].packed;
      P.w_scale = io[i].w_scale;
      P.y = io[i].y;
      P.acc_out = io[i].acc;
      P.q = qptr[i];
      P.x_scale = xsptr[i];
      P.qsum = qsptr[i];
      P.n = (int32_t)ns[i];
      P.k = (int32_t)ks[i];
      P.ldq = (int32_t)round_up(ks[i], kKPad);
      P.tiles_n = (int32_t)((ns[i] + bn - 1) / bn);
      P.ldy = (int32_t)ns[i];
      P.narrow = L.all_narrow ? 1 : 0;
      P.ksplit = L.pf_ksplit[i];
      P.kspw = L.pf_kspw[i];
      P.part = P.ksplit > 1 ? reinterpret_cast<int32_t*>(ws + L.pf_part_off[i]) : nullptr;
      P.tiled = io[i].tiled;
      P.bias = io[i].bias;
      P.res = io[i].res;
    }
    // The last tile columns of the last projection become narrow tiles when
    // that evens out the launch's last round of workgroups.
    int entries = count;
    if (load_mode == 0 && !L.all_narrow && count < kMaxProj) {
      int64_t slabs[kMaxProj], cols[kMaxProj];
      int parts[kMaxProj];
      for (int o = 0; o < count; ++o) {
        slabs[o] = pa.p[o].kspw;
        cols[o] = pa.p[o].n;
        parts[o] = pa.p[o].ksplit;
      }
      const int c = plan_narrow_columns<kPrefillBN, kPrefillNarrowBN>(
          count, slabs, cols, pa.tiles_m, (int64_t)kPrefillWgsPerCu * device_cu_count(), parts);
      if (c > 0) {
        PrefillProj& W = pa.p[count - 1];
        const int32_t keep = (W.tiles_n - c) * kPrefillBN;  // columns that stay in wide tiles
        PrefillProj T = W;
        T.packed = W.packed + (int64_t)keep * (W.k / 4);
        T.y = W.y ? W.y + keep : nullptr;
        T.acc_out = W.acc_out ? W.acc_out + keep : nullptr;
        T.bias = W.bias ? W.bias + keep : nullptr;
        T.res = W.res ? W.res + keep : nullptr;
        T.n = W.n - keep;
        T.tiles_n = (T.n + kPrefillNarrowBN - 1) / kPrefillNarrowBN;
        T.narrow = 1;
        if (keep == 0) {
          W = T;
        } else {
          W.n = keep;
          W.tiles_n -= c;
          pa.p[count] = T;
          entries = count + 1;
        }
      }
    }
    pa.count = entries;
    int64_t tiles = 0, pieces = 0;
    for (int o = 0; o < entries; ++o) {
      const PrefillProj& P = pa.p[o];
      pa.tile_begin[o] = (int32_t)tiles;
      tiles += round_up((int64_t)pa.tiles_m * P.tiles_n * P.ksplit, 8);  // XCD-aligned ranges
      pa.fin_begin[o] = (int32_t)pieces;
      if (P.ksplit > 1) pieces += m * ((P.n + 7) / 8);  // 8 outputs of one row each
    }
    for (int o = entries; o < kMaxProj; ++o) {
      pa.tile_begin[o] = (int32_t)tiles;
      pa.fin_begin[o] = (int32_t)pieces;
    }
    if (tiles >= (int64_t(1) << 31) || pieces >= (int64_t(1) << 31)) return BL_ESHAPE;
    if (launch_prefill(pa, (int)tiles, stream) != hipSuccess) return BL_EHIP;
    if (launch_prefill_finish(pa, (int)pieces, stream) != hipSuccess) return BL_EHIP;
  }
  return BL_OK;
}

// Device memory of bitlinear_forward_grouped_noalloc: a fixed array in the
// code object, so that call needs no allocation.  Each GPU the library runs
// on holds its own copy for the life of the process.  Its host-side name is
// only a stand-in for registration: kernels get the device address that
// hipGetSymbolAddress reports for the current device.
constexpr size_t kScratchBytes = (size_t)BL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current; nullptr on failure.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* bitlinear_status_string(bl_status s) {
  switch (s) {
    case BL_OK: return "ok";
    case BL_EINVAL: return "invalid argument (null pointer or count out of range)";
    case BL_ESHAPE:
      return "unsupported shape (M, N, K >= 1, K % 4 == 0, K <= 2^22; tiled weights: "
             "N % 16 == 0, K % 256 == 0)";
    case BL_EALIGN: return "pointer not 16-byte aligned";
    case BL_EWORKSPACE: return "workspace missing or too small";
    case BL_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int bitlinear_abi_version(void) { return 4; }

size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k) {
  (void)n;
  (void)k;
  return kPackWorkspace;
}

bl_status bitlinear_pack_weights(const float* w, int64_t n, int64_t k, uint8_t* packed,
                                 float* w_scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  bl_status st;
  if ((st = check_shape(1, n, k)) != BL_OK) return st;
  if (n * k >= kMaxElems) return BL_ESHAPE;
  if ((st = check_ptr(w)) != BL_OK || (st = check_ptr(packed)) != BL_OK) return st;
  if ((st = check_ptr(w_scale)) != BL_OK) return st;
  if (!workspace || workspace_bytes < kPackWorkspace) return BL_EWORKSPACE;
  if (!aligned16(workspace)) return BL_EALIGN;
  if (launch_pack(w, n, k, packed, w_scale, static_cast<unsigned long long*>(workspace),
                  static_cast<hipStream_t>(stream)) != hipSuccess)
    return BL_EHIP;
  return BL_OK;
}

bl_status bitlinear_export_bf16(const uint8_t* packed, int64_t n, int64_t k, int32_t layout,
                                const float* w_scale, uint16_t* out, void* stream) {
  bl_status st;
  if ((st = check_shape(1, n, k)) != BL_OK) return st;
  if (n * k >= kMaxElems) return BL_ESHAPE;
  if (layout != BL_LAYOUT_ROWS && layout != BL_LAYOUT_TILED) return BL_EINVAL;
  if (layout == BL_LAYOUT_TILED && (st = check_tiled_shape(n, k)) != BL_OK) return st;
  if ((st = check_ptr(packed)) != BL_OK || (st = check_ptr(w_scale)) != BL_OK ||
      (st = check_ptr(out)) != BL_OK)
    return st;
  if (launch_export_bf16(packed, n, k, layout == BL_LAYOUT_TILED, w_scale, out,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return BL_EHIP;
  return BL_OK;
}

bl_status bitlinear_unpack_weights(const uint8_t* packed, int64_t n, int64_t k, int8_t* u,
                                   void* stream) {
  bl_status st;
  if ((st = check_shape(1, n, k)) != BL_OK) return st;
  if ((st = check_ptr(packed)) != BL_OK || (st = check_ptr(u)) != BL_OK) return st;
  if (launch_unpack(packed, n, k, u, static_cast<hipStream_t>(stream)) != hipSuccess)
    return BL_EHIP;
  return BL_OK;
}

static bl_status retile(const uint8_t* src, int64_t n, int64_t k, uint8_t* dst, bool untile,
                        void* stream) {
  bl_status st;
  if ((st = check_shape(1, n, k)) != BL_OK || (st = check_tiled_shape(n, k)) != BL_OK) return st;
  if ((st = check_ptr(src)) != BL_OK || (st = check_ptr(dst)) != BL_OK) return st;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t bytes = (uintptr_t)(n * (k / 4));
  if (a < b + bytes && b < a + bytes) return BL_EINVAL;  // overlapping arrays
  if (launch_tile(src, n, k, dst, untile, static_cast<hipStream_t>(stream)) != hipSuccess)
    return BL_EHIP;
  return BL_OK;
}

bl_status bitlinear_tile_weights(const uint8_t* packed, int64_t n, int64_t k, uint8_t* tiled,
                                 void* stream) {
  return retile(packed, n, k, tiled, false, stream);
}

bl_status bitlinear_untile_weights(const uint8_t* tiled, int64_t n, int64_t k, uint8_t* packed,
                                   void* stream) {
  return retile(tiled, n, k, packed, true, stream);
}

bl_status bitlinear_act_quant(const uint16_t* x, int64_t m, int64_t k, int8_t* q,
                              float* x_scale, void* stream) {
  bl_status st;
  if ((st = check_shape(m, 1, k)) != BL_OK) return st;
  if ((st = check_ptr(x)) != BL_OK || (st = check_ptr(q)) != BL_OK ||
      (st = check_ptr(x_scale)) != BL_OK)
    return st;
  if (launch_act_quant_public(x, m, k, q, x_scale, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return BL_EHIP;
  return BL_OK;
}

size_t bitlinear_forward_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (check_shape(m, n, k) != BL_OK) return 0;
  Layout L;
  make_layout(1, &n, &k, m, false, L);  // also covers bitlinear_forward_acc
  return L.total;
}

static bl_status forward_one(int64_t m, int64_t n, int64_t k, const uint16_t* x,
                             const uint8_t* packed, const float* w_scale, uint16_t* y,
                             void* workspace, size_t workspace_bytes, void* stream, int tiled) {
  bl_status st;
  if ((st = check_shape(m, n, k)) != BL_OK) return st;
  if (tiled && (st = check_tiled_shape(n, k)) != BL_OK) return st;
  if ((st = check_ptr(x)) != BL_OK || (st = check_ptr(packed)) != BL_OK ||
      (st = check_ptr(w_scale)) != BL_OK || (st = check_ptr(y)) != BL_OK)
    return st;
  ProjIO io = {x, nullptr, packed, w_scale, y, nullptr, n, k, tiled,
               nullptr, nullptr, nullptr, nullptr, nullptr};
  return run_forward(1, &io, m, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

bl_status bitlinear_forward(int64_t m, int64_t n, int64_t k, const uint16_t* x,
                            const uint8_t* packed, const float* w_scale, uint16_t* y,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return forward_one(m, n, k, x, packed, w_scale, y, workspace, workspace_bytes, stream, 0);
}

bl_status bitlinear_forward_tiled(int64_t m, int64_t n, int64_t k, const uint16_t* x,
                                  const uint8_t* tiled, const float* w_scale, uint16_t* y,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return forward_one(m, n, k, x, tiled, w_scale, y, workspace, workspace_bytes, stream, 1);
}

size_t bitlinear_forward_grouped_workspace_bytes(int32_t count, const bl_projection* projs,
                                                 int64_t m) {
  if (count < 1 || count > kMaxProj || !projs) return 0;
  int64_t ns[kMaxProj], ks[kMaxProj];
  for (int i = 0; i < count; ++i) {
    if (check_shape(m, projs[i].n, projs[i].k) != BL_OK) return 0;
    ns[i] = projs[i].n;
    ks[i] = projs[i].k;
  }
  Layout L;
  make_layout(count, ns, ks, m, false, L);
  return L.total;
}

static bl_status grouped_io(int32_t count, const bl_projection* projs, int64_t m, ProjIO* io) {
  if (count < 1 || count > kMaxProj || !projs) return BL_EINVAL;
  for (int i = 0; i < count; ++i) {
    const bl_projection& p = projs[i];
    bl_status st;
    if ((st = check_shape(m, p.n, p.k)) != BL_OK) return st;
    if ((p.layout != BL_LAYOUT_ROWS && p.layout != BL_LAYOUT_TILED) || p.reserved != 0)
      return BL_EINVAL;
    if (p.layout == BL_LAYOUT_TILED && (st = check_tiled_shape(p.n, p.k)) != BL_OK) return st;
    if ((st = check_ptr(p.x)) != BL_OK || (st = check_ptr(p.packed)) != BL_OK ||
        (st = check_ptr(p.w_scale)) != BL_OK || (st = check_ptr(p.y)) != BL_OK)
      return st;
    if ((p.bias && !aligned16(p.bias)) || (p.residual && !aligned16(p.residual))) return BL_EALIGN;
    if (p.residual && p.residual != p.y) {  // in place, or apart
      const uintptr_t a = reinterpret_cast<uintptr_t>(p.residual);
      const uintptr_t b = reinterpret_cast<uintptr_t>(p.y);
      const uintptr_t bytes = (uintptr_t)(m * p.n) * 2;
      if (a < b + bytes && b < a + bytes) return BL_EINVAL;
    }
    io[i] = ProjIO{p.x,     nullptr, p.packed, p.w_scale, p.y,    nullptr,
                   p.n,     p.k,     p.layout == BL_LAYOUT_TILED ? 1 : 0,   nullptr, nullptr,
                   nullptr, p.bias,  p.residual};
  }
  return BL_OK;
}

int32_t bitlinear_forward_grouped_launches(int32_t count, const bl_projection* projs, int64_t m) {
  if (count < 1 || count > kMaxProj || !projs) return -1;
  int64_t ns[kMaxProj], ks[kMaxProj];
  for (int i = 0; i < count; ++i) {
    if (check_shape(m, projs[i].n, projs[i].k) != BL_OK) return -1;
    ns[i] = projs[i].n;
    ks[i] = projs[i].k;
  }
  Layout L;
  make_layout(count, ns, ks, m, true, L);  // bf16 activations, as the grouped call takes
  int jobs = 0;
  for (int i = 0; i < count; ++i) jobs += (L.decode && L.plan[i].fused) ? 0 : 1;
  int32_t launches = (jobs > 0 || L.zero_bytes > 0) ? 1 : 0;  // activation quantization
  launches += 1;                                              // the contraction
  if (!L.decode)
    for (int i = 0; i < count; ++i)
      if (L.pf_ksplit[i] > 1) {  // the pass that adds the K parts
        launches += 1;
        break;
      }
  return launches;
}

bl_status bitlinear_forward_grouped(int32_t count, const bl_projection* projs, int64_t m,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  ProjIO io[kMaxProj];
  const bl_status st = grouped_io(count, projs, m, io);
  if (st != BL_OK) return st;
  return run_forward(count, io, m, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

bl_status bitlinear_forward_grouped_noalloc(int32_t count, const bl_projection* projs, int64_t m,
                                            void* stream) {
  ProjIO io[kMaxProj];
  const bl_status st = grouped_io(count, projs, m, io);
  if (st != BL_OK) return st;
  int64_t ns[kMaxProj], ks[kMaxProj];
  for (int i = 0; i < count; ++i) {
    ns[i] = io[i].n;
    ks[i] = io[i].k;
  }
  Layout L;
  make_layout(count, ns, ks, m, false, L);
  if (L.total > kScratchBytes) return BL_EWORKSPACE;
  void* ws = scratch_address();
  if (!ws) return BL_EHIP;
  return run_forward(count, io, m, ws, kScratchBytes, static_cast<hipStream_t>(stream));
}

bl_status bitlinear_forward_grouped_inspect(int32_t count, const bl_projection* projs, int64_t m,
                                            const bl_inspect* inspect, int32_t* status,
                                            int32_t wait_polls, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  ProjIO io[kMaxProj];
  bl_status st = grouped_io(count, projs, m, io);
  if (st != BL_OK) return st;
  if (!inspect) return BL_EINVAL;
  if (status && (st = check_ptr(status)) != BL_OK) return st;
  for (int i = 0; i < count; ++i) {
    const bl_inspect& d = inspect[i];
    // optional outputs: 16-byte aligned when given
    for (const void* p : {(const void*)d.q, (const void*)d.x_scale, (const void*)d.qsum,
                          (const void*)d.acc})
      if (p && !aligned16(p)) return BL_EALIGN;
    io[i].ins_q = d.q;
    io[i].ins_xs = d.x_scale;
    io[i].ins_qs = d.qsum;
    io[i].acc = d.acc;
  }
  CallDiag diag;
  diag.status = status;
  diag.wait_polls = wait_polls > 0 ? wait_polls : (wait_polls == 0 ? kDefaultWaitPolls : 0);
  return run_forward(count, io, m, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                     diag);
}

// Workspace of bitlinear_forward_latent: the absmean buckets, the weight
// scale, the packed weights, then a forward call's workspace.
struct LatentLayout {
  size_t scale, packed, fwd, total;
};

static LatentLayout latent_layout(int64_t m, int64_t n, int64_t k) {
  LatentLayout L;
  L.scale = align256(kPackWorkspace);
  L.packed = align256(L.scale + sizeof(float));
  L.fwd = align256(L.packed + (size_t)n * (size_t)(k / 4));
  Layout F;
  make_layout(1, &n, &k, m, false, F);
  L.total = L.fwd + F.total;
  return L;
}

size_t bitlinear_forward_latent_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (check_shape(m, n, k) != BL_OK || n * k >= kMaxElems) return 0;
  return latent_layout(m, n, k).total;
}

bl_status bitlinear_forward_latent(int64_t m, int64_t n, int64_t k, const uint16_t* x,
                                   const float* w, float* w_scale, uint16_t* y, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  bl_status st;
  if ((st = check_shape(m, n, k)) != BL_OK) return st;
  if (n * k >= kMaxElems) return BL_ESHAPE;
  if ((st = check_ptr(x)) != BL_OK || (st = check_ptr(w)) != BL_OK || (st = check_ptr(y)) != BL_OK)
    return st;
  if (w_scale && !aligned16(w_scale)) return BL_EALIGN;
  const LatentLayout L = latent_layout(m, n, k);
  if (!workspace) return BL_EWORKSPACE;
  if (!aligned16(workspace)) return BL_EALIGN;
  if (workspace_bytes < L.total) return BL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* scale = w_scale ? w_scale : reinterpret_cast<float*>(ws + L.scale);
  uint8_t* packed = reinterpret_cast<uint8_t*>(ws + L.packed);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // stage 1: the exact global absmean; stage 2: block-wise ternarization and
  // packing; then the forward pass on the packed weights
  if (launch_pack(w, n, k, packed, scale, reinterpret_cast<unsigned long long*>(ws), s) !=
      hipSuccess)
    return BL_EHIP;
  ProjIO io = {x, nullptr, packed, scale, y, nullptr, n, k, 0,
               nullptr, nullptr, nullptr, nullptr, nullptr};
  return run_forward(1, &io, m, ws + L.fwd, workspace_bytes - L.fwd, s);
}

static bl_status forward_acc_one(int64_t m, int64_t n, int64_t k, const int8_t* q,
                                 const uint8_t* packed, int32_t* acc, void* workspace,
                                 size_t workspace_bytes, void* stream, int tiled) {
  bl_status st;
  if ((st = check_shape(m, n, k)) != BL_OK) return st;
  if (tiled && (st = check_tiled_shape(n, k)) != BL_OK) return st;
  if ((st = check_ptr(q)) != BL_OK || (st = check_ptr(packed)) != BL_OK ||
      (st = check_ptr(acc)) != BL_OK)
    return st;
  ProjIO io = {nullptr, q, packed, nullptr, nullptr, acc, n, k, tiled,
               nullptr, nullptr, nullptr, nullptr, nullptr};
  return run_forward(1, &io, m, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

bl_status bitlinear_forward_acc(int64_t m, int64_t n, int64_t k, const int8_t* q,
                                const uint8_t* packed, int32_t* acc, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return forward_acc_one(m, n, k, q, packed, acc, workspace, workspace_bytes, stream, 0);
}

bl_status bitlinear_forward_acc_tiled(int64_t m, int64_t n, int64_t k, const int8_t* q,
                                      const uint8_t* tiled, int32_t* acc, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return forward_acc_one(m, n, k, q, tiled, acc, workspace, workspace_bytes, stream, 1);
}

}  // extern "C"
