// Decode path, host side: the launch planners and the launches of the
// decode kernel (decode_kernels.hpp).  The instances for 2-8 token rows with
// fused activation quantization are compiled in decode_fused.hip.
#include "decode_kernels.hpp"

namespace bl {

// Work split of one projection.  The K range of a WG is limited by the LDS
// budget for staged codes (beyond it WGs split K and add partial sums in
// L2).  Waves of a WG split K as well when its range is long (1, 2 or 4
// ways, partial sums meet in LDS); otherwise each wave owns its own row
// tiles.  Tiles per wave bring a wave's stream to about `target` 16-byte
// chunks (a WG moves about 64 KB at the default target).  Small M*K with 16-aligned rows takes
// the fused path (the WG quantizes the bf16 rows itself), which never
// splits K across WGs.
DecodePlan plan_decode(int64_t m, int64_t n, int64_t k, int mode, int target) {
  DecodePlan p;
  const int S = (int)((k + 255) / 256);
  int cap = (int)((kDecodeLdsA / m - 16) / 256);
  if (cap < 1) cap = 1;
  if (cap > 4 * kWaveMaxChunks) cap = 4 * kWaveMaxChunks;
  p.ksplit = (S + cap - 1) / cap;
  p.kspw = (S + p.ksplit - 1) / p.ksplit;
  p.wk = p.kspw <= target ? 1 : (p.kspw <= 2 * kWaveMaxChunks ? 2 : 4);
  if (p.wk == 2 && (p.kspw + 1) / 2 > target && p.kspw > 2 * target) p.wk = 4;
  const int nsw = (p.kspw + p.wk - 1) / p.wk;  // <= kWaveMaxChunks
  int tww = 1;
  while (tww < kDecodeMaxTww && 2 * tww * nsw <= target) tww *= 2;  // 1, 2 or 4
  const int rows_wg = (4 / p.wk) * tww * 16;
  p.tww = tww;
  p.ngroups = (int)((n + rows_wg - 1) / rows_wg);
  p.fused = mode == 0 && m <= kFusedMaxM && k % 16 == 0 && m * k <= fused_max_elems(m) &&
            p.ksplit == 1;
  return p;
}

// Split-shape plan for a whole layer: one workgroup per CU at most, each
// streaming wave's share as small as possible.  Per projection the choice is
// the K split over the 4 streaming waves (wk) and the 16-row tiles per wave
// (tww, 1-4); a wave then streams tww * ceil(S / wk) 16-byte chunks per lane
// (S = 256-code slabs per row).  The smallest bound X on that count for which
// the fewest workgroups each projection needs add up to at most `cus` wins.
// K is never split across workgroups here, so every row's codes fit LDS.
bool plan_decode_split(int64_t m, int32_t count, const int64_t* ns, const int64_t* ks, int mode,
                       int cus, bool have_x, DecodePlan* plans) {
  constexpr int kMaxChunks = 96;  // per lane: at most six rounds of the ring
  constexpr int kSplitPlanMinChunks = 48;
  constexpr int kSmallLayerCuShare = 4;  // "most CUs idle": a quarter of them or fewer busy
  if (mode != 0 || count < 1 || count > kMaxProj) return false;
  int S[kMaxProj];
  int64_t tiles[kMaxProj];
  bool fuse[kMaxProj];
  for (int i = 0; i < count; ++i) {
    S[i] = (int)((ks[i] + 255) / 256);
    tiles[i] = (ns[i] + 15) / 16;
    // rows the kernel quantizes itself may use the split plan's larger code
    // budget; staged codes are loaded in at most kDecodeLdsA bytes
    fuse[i] = have_x && m <= kFusedMaxM && ks[i] % 16 == 0 && m * ks[i] <= fused_max_elems(m, true);
    if (m * (S[i] * 256 + 16) > (fuse[i] ? kDecodeSplitLdsA : kDecodeLdsA)) return false;
  }
  // (wk, tww) pairs; seven tiles per wave with two waves per K range lets
  // the 8B-class layer's longest wave stream 56 chunks on 240 CUs instead of
  // 64 on 216
  constexpr int kOpts = 11;
  const int wks[kOpts] = {1, 1, 1, 1, 2, 2, 2, 2, 4, 4, 4};
  const int twws[kOpts] = {1, 2, 3, 4, 1, 2, 4, 7, 1, 2, 4};
  for (int x = 1; x <= kMaxChunks; ++x) {
    int64_t total = 0;
    bool ok = true;
    for (int i = 0; i < count && ok; ++i) {
      int64_t best = -1;
      for (int o = 0; o < kOpts; ++o) {
        const int wk = wks[o], tww = twws[o];
        if (tww * ((S[i] + wk - 1) / wk) > x) continue;
        const int64_t per = (int64_t)(4 / wk) * tww;  // 16-row tiles per workgroup
        const int64_t wgs = (tiles[i] + per - 1) / per;
        if (best < 0 || wgs < best) {
          best = wgs;
          DecodePlan& p = plans[i];
          p.wk = wk;
          p.tww = tww;
          p.kspw = S[i];
          p.ksplit = 1;
          p.ngroups = (int)wgs;
          p.fused = fuse[i];
        }
      }
      if (best < 0) ok = false;
      total += best;
    }
    // Shorter streams are left to the per-projection plans: measured on
    // the 3B-class layer (36 chunks per wave here) the many-workgroup ring
    // shape was faster, on the 8B-class layer (64) this plan was.  Except
    // when those plans would leave most CUs idle (a small layer: a single
    // 2048 x 2048 projection at M = 8 takes 16 workgroups of 64 KB, against
    // 128 of 8 KB here; measured 10.8 -> 8.9 us per call).
    if (ok && total <= cus) {
      if (x >= kSplitPlanMinChunks) return true;
      int64_t own = 0;
      for (int i = 0; i < count; ++i) {
        const DecodePlan q = plan_decode(m, ns[i], ks[i], mode);
        own += (int64_t)q.ngroups * q.ksplit;
      }
      return own * kSmallLayerCuShare <= cus;
    }
  }
  return false;
}

int current_device_index() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  return dev;
}

int device_cu_count() {
  static int cus[kMaxDevices] = {0};
  const int dev = current_device_index();
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 1;
    cus[dev] = n > 0 ? n : 1;
  }
  return cus[dev];
}

size_t decode_lds_bytes(int64_t m, int lds_row) {
  return (size_t)m * lds_row + (size_t)4 * kDecodeRedTww * m * 16 * 4;
}

hipError_t launch_decode(const DecodeArgs& a, int total_wgs, size_t lds_bytes, hipStream_t s) {
  // extra epilogue work: int32 accumulators next to bf16 outputs, the fused
  // quantization's codes, scales or code sums, a bias or a residual
  bool ins = false;
  for (int i = 0; i < a.count; ++i) {
    const DecodeProj& P = a.p[i];
    ins = ins || (P.y && P.acc_out) || (P.x && (P.q || P.x_scale || P.qsum)) || a.epi[i].bias ||
          a.epi[i].res;
  }
  bool fused = false, big = false;
  for (int i = 0; i < a.count; ++i) {
    fused = fused || a.p[i].x;
    big = big || (a.p[i].x && (int64_t)a.m * a.p[i].k > fused_max_elems(a.m));
  }
  if (fused && a.m > 1) return launch_decode_rows(a, total_wgs, lds_bytes, s, ins, big);
  if (fused)  // one token row
    return ins ? launch_decode_as<true, 1>(a, total_wgs, lds_bytes, s)
               : launch_decode_as<false, 1>(a, total_wgs, lds_bytes, s);
  return ins ? launch_decode_as<true, 0>(a, total_wgs, lds_bytes, s)
             : launch_decode_as<false, 0>(a, total_wgs, lds_bytes, s);
}

}  // namespace bl
