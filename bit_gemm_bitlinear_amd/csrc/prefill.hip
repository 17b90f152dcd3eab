// Prefill contraction (M > 16 tokens) on the int8 matrix cores:
// acc[m][n] = sum_k q[m][k] * u[n][k], then y = bf16(acc / (x_scale[m] *
// w_scale)) -- F.linear and post_quant_process of BitLinear.forward in the
// Falcon-Edge blog ("A series of powerful, universal and fine-tunable 1.58-bit
// language models", section "Falcon-Edge, a series of universal models").
//
// A dense contraction, so it runs on v_mfma_i32_32x32x32_i8 (half the
// operand bytes and half the weight-expansion work per multiply of the
// 16x16x64 form).  Two variants:
//  * the main one (prefill_kernel, "Main variant" below) for weight rows that
//    are 16-byte aligned (K % 64 == 0): both operands go from global memory
//    straight into LDS, slabs of 128 codes, two workgroups per CU;
//  * the register-staged one (prefill_reg_kernel, next) for other K.
//
// Register-staged variant: a workgroup computes a 128 (tokens) x 256
// (outputs) tile with four waves of 64 x 128 (2 x 4 matrix-core tiles of
// 32 x 32).
//  * K advances by slabs of 256 codes.  The activation-code tile of a slab
//    (128 rows x 256 B, internal layout from act_quant.hip) is staged in LDS,
//    double-buffered: slab s+1 is fetched into registers while slab s is
//    consumed, then written to the other buffer.  16-byte chunk c of row r is
//    stored at chunk c ^ (r & 15), which spreads the rows one A fragment
//    reads over all banks.
//  * Packed weights are small (2 bits each) and each wave needs its own 128
//    columns, so they go straight from global memory to registers, one slab
//    ahead, and are expanded there (common.hpp).  In K-step s of a slab, lane
//    (column j, half g) supplies codes 128g + 16s .. +15, i.e. 32 contiguous
//    packed bytes per lane per slab; the activation fragment uses the same
//    codes (the assignment of codes to K-steps is free as long as both
//    operands agree).
//  * Rows of codes are zero-padded to the tile, K to 256, so activation loads
//    need no bounds checks; weight rows and columns past the end are clamped
//    to valid addresses (they meet zero codes or reach outputs that are not
//    stored).
#include "common.hpp"
#include "internal.hpp"

#include <atomic>
#include <type_traits>

namespace bl {

namespace {

constexpr int kThreads = 256;
constexpr int BM = kPrefillBM;  // 128
constexpr int BN = kPrefillRegBN;  // 256 (register-staged variant)
constexpr int kStageChunks = BM * 16 / kThreads;  // 16-byte A chunks per thread per slab

typedef int32_t v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16i mfma_32x32x32_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// 16 bytes of a packed row (see decode.hip); MODE fixes the row alignment.
template <int MODE>
__device__ __forceinline__ v4i load_w16(const uint8_t* __restrict__ row, int off, int rowbytes) {
  v4i r;
  if constexpr (MODE == 0) {
    r = *G(reinterpret_cast<const v4i*>(row + min(off, rowbytes - 16)));
  } else if constexpr (MODE == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = *G(reinterpret_cast<const int32_t*>(row + min(off + 4 * j, rowbytes - 4)));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t d = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) d |= (uint32_t)*G(row + min(off + 4 * j + b, rowbytes - 1)) << (8 * b);
      r[j] = (int32_t)d;
    }
  }
  return r;
}

struct Tile {
  const PrefillProj* P;
  int m0, n0;
};

// Weight fragments of one slab: 4 column tiles x 32 packed bytes per lane.
template <int MODE>
__device__ __forceinline__ void load_b(v4i (&b)[4][2], const PrefillProj& P, int ncol0, int slab,
                                       int lj, int lg) {
  const int rowbytes = P.k >> 2;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int row = min(ncol0 + 32 * f + lj, P.n - 1);
    const int off = slab * 64 + 32 * lg;
    if (P.tiled) {  // 64-byte aligned rows: two whole chunks (common.hpp)
      b[f][0] = *G(reinterpret_cast<const v4i*>(P.packed + tiled_chunk_offset(row, off, rowbytes)));
      b[f][1] = *G(reinterpret_cast<const v4i*>(P.packed + tiled_chunk_offset(row, off + 16, rowbytes)));
    } else {
      const uint8_t* rp = P.packed + (int64_t)row * rowbytes;
      b[f][0] = load_w16<MODE>(rp, off, rowbytes);
      b[f][1] = load_w16<MODE>(rp, off + 16, rowbytes);
    }
  }
}

__device__ __forceinline__ void load_a(v4i (&st)[kStageChunks], const PrefillProj& P, int m0,
                                       int slab) {
#pragma unroll
  for (int i = 0; i < kStageChunks; ++i) {
    const int id = threadIdx.x + kThreads * i;
    const int r = id >> 4, c = id & 15;
    st[i] = *G(reinterpret_cast<const v4i*>(P.q + (int64_t)(m0 + r) * P.ldq + slab * 256 + 16 * c));
  }
}

__device__ __forceinline__ void store_a(int8_t* __restrict__ buf, const v4i (&st)[kStageChunks]) {
#pragma unroll
  for (int i = 0; i < kStageChunks; ++i) {
    const int id = threadIdx.x + kThreads * i;
    const int r = id >> 4, c = id & 15;
    *reinterpret_cast<v4i*>(buf + r * 256 + 16 * (c ^ (r & 15))) = st[i];
  }
}

// Tile of workgroup `l` of a projection, by XCD.  Workgroups go to the 8
// XCDs round-robin (l % 8, each projection's range starts at a multiple of
// 8) and every XCD has its own L2, so each XCD gets one contiguous share of
// the tiles: when the M-tile count is a multiple of 8, a share is whole
// M-tiles walked N-outer (its activation rows stay in its L2 and
// neighbouring workgroups reuse each weight tile); otherwise a share is a
// contiguous range of N-tiles (its weights are read by no other XCD).
// Returns false for padding workgroups.
__device__ __forceinline__ bool tile_of(int l, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int T = tiles_m * tiles_n;
  const int chunk = (T + 7) >> 3;
  const int x = l & 7, w = l >> 3;
  if (w >= chunk) return false;
  if ((tiles_m & 7) == 0) {
    const int mt = tiles_m >> 3;
    *tm = x * mt + w % mt;
    *tn = w / mt;
    return true;
  }
  const int L = x * chunk + w;
  if (L >= T) return false;
  *tm = L % tiles_m;
  *tn = L / tiles_m;
  return true;
}

// Register-staged variant (weight rows not 16-byte aligned): activation codes
// through a double-buffered LDS tile, weights straight to registers.
template <int MODE>
__global__ __launch_bounds__(kThreads) void prefill_reg_kernel(const PrefillArgs A) {
  __shared__ __align__(16) int8_t abuf[2][BM * 256];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i) pi += (i < A.count && (int)blockIdx.x >= A.tile_begin[i]);
  const PrefillProj& P = A.p[pi];
  int tm, tn;
  if (!tile_of((int)blockIdx.x - A.tile_begin[pi], A.tiles_m, P.tiles_n, &tm, &tn)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lj = lane & 31, lg = lane >> 5;
  const int m0 = tm * BM;
  const int wm0 = (wave & 1) * 64;              // wave's rows within the tile
  const int ncol0 = tn * BN + (wave >> 1) * 128;  // wave's first output column
  const int S = (P.k + 255) >> 8;
  __shared__ int32_t s_qs[BM];
  __shared__ RowDiv s_rd[BM];
  if (tid < BM && m0 + tid < A.m) {
    s_qs[tid] = *G(P.qsum + m0 + tid);
    if (P.y) s_rd[tid] = row_div_setup(*G(P.x_scale + m0 + tid) * *C(P.w_scale));
  }

  v16i acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0;

  v4i st[kStageChunks];
  v4i bcur[4][2], bnext[4][2];
  load_a(st, P, m0, 0);
  load_b<MODE>(bcur, P, ncol0, 0, lj, lg);
  store_a(abuf[0], st);
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    const bool more = s + 1 < S;
    if (more) {
      load_a(st, P, m0, s + 1);
      load_b<MODE>(bnext, P, ncol0, s + 1, lj, lg);
    }
    const int8_t* buf = abuf[s & 1];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      // this lane's 16 codes of K-step ks: chunk 8g + ks of its rows
      v4i a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm0 + 32 * i + lj;
        a[i] = *reinterpret_cast<const v4i*>(buf + r * 256 + 16 * ((8 * lg + ks) ^ (r & 15)));
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const v4i bq = decode16((uint32_t)bcur[f][ks >> 2][ks & 3]);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][f] = mfma_32x32x32_i8(a[i], bq, acc[i][f]);
      }
    }
    if (more) store_a(abuf[(s + 1) & 1], st);
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      bcur[f][0] = bnext[f][0];
      bcur[f][1] = bnext[f][1];
    }
  }

  // epilogue: lane holds C[8*(r/4) + 4*lg + r%4][lj] of each 32x32 tile
  // (the loop's last barrier also published s_qs / s_rd)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = wm0 + 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
      const int m = m0 + ml;
      if (m >= A.m) continue;
      const int32_t qs = s_qs[ml];
      const RowDiv rd = s_rd[ml];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int n = ncol0 + 32 * f + lj;
        if (n >= P.n) continue;
        const int32_t v = acc[i][f][r] - qs;
        if (P.y) {
          uint16_t yb = dequant_bf16_row(v, rd);
          if (P.bias) yb = add_bf16(yb, *G(P.bias + n));
          if (P.res) yb = add_bf16(yb, *G(P.res + (int64_t)m * P.ldy + n));
          *G(P.y + (int64_t)m * P.ldy + n) = yb;
        }
        if (P.acc_out) *G(P.acc_out + (int64_t)m * P.ldy + n) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Main variant (16-byte aligned weight rows): both operands of a slab go
// straight from global memory into LDS (gfx950 global_load_lds, 16 bytes
// per lane, lane L's bytes landing at dst + 16 L), through a ring of NST
// slab buffers: while slab s is multiplied, slabs up to s+NST-1 are in
// flight.  No staging registers, one barrier per slab.  The tile is TBM
// tokens (128; 32 or 64 in the mid-M range, prefill_bm) x BNT outputs (256, or
// 128 for the entries the host marks narrow); a slab is BK codes deep (128 or
// 256).  The expanded weights are the matrix
// core's first operand and the activation codes its second, so each lane's
// sums belong to one token row (see the epilogue).
//
// LDS image of a slab (KA = BK/16 chunks of 16 B per A row, KB = BK/64 per
// B column):
//   A: 128 rows x KA chunks; chunk c of row r at r*KA + (c ^ ((r / (16/KA)) & (KA-1))).
//   B: BNT columns x KB chunks (16 packed bytes = 64 codes each); chunk c of
//      column j at j*KB + (c ^ ((j / (16/KB)) & (KB-1))).
// Both swizzles keep the 16 lanes that LDS serves together on distinct banks.  The two
// halves of a wave (lanes 0-31, 32-63) take the two halves of the slab's K
// range, so one matrix-core step pairs A chunks ks and KA/2 + ks with
// packed B dword ks of the lane's B chunk.

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits until at most `ahead` slabs of D loads each are still in flight
// (ahead <= C; a compile-time count per case, as the wait needs one).
template <int D, int C>
__device__ __forceinline__ void wait_slabs(int ahead) {
  if constexpr (C == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= C)
      wait_vm<C * D>();
    else
      wait_slabs<D, C - 1>(ahead);
  }
}

__device__ __forceinline__ void dma16(const void* src, int8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((const BL_GLOBAL void*)src,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

template <int BNT, int WMI, int NW, int BK, int TBM>
struct Cfg {
  static_assert(BK == 128 || BK == 256, "a slab is 128 or 256 codes deep");
  static constexpr int kNT = 64 * NW;  // threads
  static constexpr int kACh = BK / 16;  // 16-byte A chunks per row of a slab
  static constexpr int kBCh = BK / 64;  // 16-byte B chunks per column of a slab
  static constexpr int kBL = kBCh / 2;  // B chunks per lane (two lane halves split K)
  static constexpr int kKS = BK / 32;   // matrix-core steps per slab
  // LDS serves a 16-byte read 16 lanes at a time from 64 banks (256 bytes):
  // the swizzles below give the 16 rows (A) or columns (B) that one such
  // group reads 16 distinct 16-byte bank slots
  static constexpr int kARowsPerSlot = 16 / kACh;  // rows sharing a swizzle value
  static constexpr int kBColsPerSlot = 16 / kBCh;
  static __device__ __forceinline__ int aswz(int r, int c) {
    return c ^ ((r / kARowsPerSlot) & (kACh - 1));
  }
  static __device__ __forceinline__ int bswz(int j, int c) {
    return c ^ ((j / kBColsPerSlot) & (kBCh - 1));
  }
  static constexpr int kAChunks = TBM * kACh;
  static constexpr int kBChunks = BNT * kBCh;
  static constexpr int kStageBytes = (kAChunks + kBChunks) * 16;
  static constexpr int kADma = kAChunks / kNT;
  static constexpr int kBDma = kBChunks / kNT;
  static constexpr int kDma = kADma + kBDma;    // DMA instructions per thread per slab
  static constexpr int kWavesM = TBM / (32 * WMI);  // waves along the tile's rows
  static constexpr int kWavesN = NW / kWavesM;     // waves along its columns
  static constexpr int WNF = BNT / (32 * kWavesN);  // 32-column tiles per wave
  static_assert(kWavesM * kWavesN == NW && WNF >= 1, "the waves cover the tile");
  static_assert(kADma * kNT == kAChunks && kBDma * kNT == kBChunks, "whole DMA blocks");
};

// The slab loads of one tile: each lane's global addresses are computed
// once per tile, so issuing a slab is an add per load.  Weight rows whose
// packed length is not a multiple of the slab's bytes have their last
// slab's loads clamped to the row (the codes there meet zero activations).
template <int BNT, int WMI, int NW, int BK, int TBM>
struct Stager {
  using K = Cfg<BNT, WMI, NW, BK, TBM>;
  const int8_t* a[K::kADma];
  const uint8_t* brow[K::kBDma];
  int bc[K::kBDma];  // byte offset of the lane's chunk within a slab of a weight row
  int rowbytes;
  int bstep;  // bytes from one slab of a weight row to the next

  __device__ __forceinline__ Stager(const PrefillProj& P, int m0, int n0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < K::kADma; ++i) {
      const int pos = (wave * K::kADma + i) * 64 + lane;
      const int r = pos / K::kACh, c = K::aswz(r, pos % K::kACh);
      a[i] = P.q + (int64_t)(m0 + r) * P.ldq + 16 * c;
    }
    rowbytes = P.k >> 2;
    // row-major: chunk c of a slab at 16 c, slabs BK/4 bytes apart.  Tiled
    // (common.hpp, k % 256 == 0): a slab of 16 rows is one contiguous run of
    // 4 * BK bytes in the rows' block, chunk c of row r at 256 c + 16 (r % 16).
    bstep = P.tiled ? 4 * BK : BK / 4;
#pragma unroll
    for (int i = 0; i < K::kBDma; ++i) {
      const int pos = (wave * K::kBDma + i) * 64 + lane;
      const int j = pos / K::kBCh, c = K::bswz(j, pos % K::kBCh);
      const int64_t r = min(n0 + j, P.n - 1);
      brow[i] = P.packed + (P.tiled ? (r >> 4) * 16 * rowbytes + 16 * (r & 15) : r * rowbytes);
      bc[i] = P.tiled ? 256 * c : 16 * c;
    }
  }

  // Slab `slab` into the stage buffer st (each instruction fills 1 KB of
  // LDS: lane L's 16 bytes land at st + 1024 * block + 16 L).
  __device__ __forceinline__ void issue(int slab, int8_t* __restrict__ st) const {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < K::kADma; ++i) dma16(a[i] + slab * BK, st + (wave * K::kADma + i) * 1024);
    int8_t* bst = st + K::kAChunks * 16;
    const int b0 = slab * (BK / 4);
    if (b0 + BK / 4 <= rowbytes) {  // always so in the tiled layout
#pragma unroll
      for (int i = 0; i < K::kBDma; ++i)
        dma16(brow[i] + slab * bstep + bc[i], bst + (wave * K::kBDma + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < K::kBDma; ++i)
        dma16(brow[i] + min(b0 + bc[i], rowbytes - 16), bst + (wave * K::kBDma + i) * 1024);
    }
  }
};

// WMI = 32-row tiles per wave.  With WMI = 4 each wave covers all 128 rows of
// the tile and its own columns, so every weight column is expanded once per
// workgroup; with WMI = 2 two waves share (and both expand) each column.
// One output tile (TBM rows x BNT columns) of projection P.
// EPI: the extra epilogue work (a separate kernel instance) -- the bias and
// then the residual added to the bf16 outputs (BitLinear.forward's bias
// line, each add rounded to bf16), and int32 accumulators written next to
// the bf16 outputs where a projection asks for both (inspection).
template <int BNT, int NST, int WMI, int NW, int BK, bool EPI, int TBM>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& A, const PrefillProj& P, int tm, int tn,
                                             int kp, int8_t* __restrict__ smem) {
  using K = Cfg<BNT, WMI, NW, BK, TBM>;
  constexpr int WNF = K::WNF;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lj = lane & 31, lg = lane >> 5;
  const int m0 = tm * TBM;
  const int n0 = tn * BNT;
  const int wm0 = (wave % K::kWavesM) * 32 * WMI;  // wave's rows within the tile
  const int wn0 = (wave / K::kWavesM) * 32 * WNF;  // wave's columns within the tile
  const int S = (P.k + BK - 1) / BK;
  const int s0 = kp * P.kspw;           // first slab of this K part
  const int nsl = min(S - s0, P.kspw);  // its slabs (all of K when unsplit)
  const bool bf = P.y != nullptr;

  // This lane's token rows, one per 32-row subtile: m0 + wm0 + 32 i + lj.
  // The accumulators start from minus the row's code sum (the contraction
  // with codes c = u + 1 then ends at the sum over q * u).
  const float ws = bf ? load_f32_vmem(P.w_scale) : 0.0f;
  float xs[WMI];
  v16i acc[WMI][WNF];
#pragma unroll
  for (int i = 0; i < WMI; ++i) {
    const int m = min(m0 + wm0 + 32 * i + lj, A.m - 1);
    const int32_t q0 = kp == 0 ? -*G(P.qsum + m) : 0;  // once per output
    xs[i] = bf ? *G(P.x_scale + m) : 1.0f;
#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = q0;
  }

  const Stager<BNT, WMI, NW, BK, TBM> stager(P, m0, n0);
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < nsl) stager.issue(s0 + p, smem + p * K::kStageBytes);

  for (int s = 0; s < nsl; ++s) {
    // wait for slab s: the slabs issued after it (at most NST-2) may still fly
    const int ahead = min(nsl - 1 - s, NST - 2);
    wait_slabs<K::kDma, NST - 2>(ahead);
    __builtin_amdgcn_s_barrier();  // every wave's slab-s data is in LDS, and
                                   // every wave is done with slab s-1's buffer
    if (s + NST - 1 < nsl)
      stager.issue(s0 + s + NST - 1, smem + ((s + NST - 1) % NST) * K::kStageBytes);
    const int8_t* abuf = smem + (s % NST) * K::kStageBytes;
    const int8_t* bbuf = abuf + K::kAChunks * 16;
    // weight chunks of this lane: column wn0 + 32f + lj, chunks kBL * lg + h
    v4i b[WNF][K::kBL];
#pragma unroll
    for (int f = 0; f < WNF; ++f) {
      const int j = wn0 + 32 * f + lj;
#pragma unroll
      for (int h = 0; h < K::kBL; ++h)
        b[f][h] = *reinterpret_cast<const v4i*>(bbuf + 16 * (j * K::kBCh + K::bswz(j, K::kBL * lg + h)));
    }
    // A fragments of step ks + 1 are read while step ks multiplies, so the
    // LDS latency hides behind the matrix-core work
    auto aload = [&](int ks, v4i (&a)[WMI]) {
#pragma unroll
      for (int i = 0; i < WMI; ++i) {
        const int r = wm0 + 32 * i + lj;
        a[i] = *reinterpret_cast<const v4i*>(abuf + 16 * (r * K::kACh + K::aswz(r, K::kKS * lg + ks)));
      }
    };
    v4i a[2][WMI];
    aload(0, a[0]);
#pragma unroll
    for (int ks = 0; ks < K::kKS; ++ks) {
      if (ks < K::kKS - 1) aload(ks + 1, a[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // the reads go out ahead of this step's work
#pragma unroll
      for (int f = 0; f < WNF; ++f) {
        const v4i bq = decode16((uint32_t)b[f][ks >> 2][ks & 3]);
#pragma unroll
        for (int i = 0; i < WMI; ++i) acc[i][f] = mfma_32x32x32_i8(bq, a[ks & 1][i], acc[i][f]);
      }
    }
  }

  // Epilogue.  The weights are the matrix core's first operand, so lane
  // (lj, lg) holds, for subtiles i and f, token row m0 + wm0 + 32 i + lj at
  // columns wn0 + 32 f + 8 a + 4 lg + b in acc[i][f][4 a + b] (a, b = 0..3):
  // runs of 4 columns of one row.  No LDS and no barrier: each lane divides
  // by its row's divisor, and for bf16 output one swap with the lane 32 away
  // turns two runs of 4 into 8 consecutive columns (a 16-byte store).
#pragma unroll
  for (int i = 0; i < WMI; ++i) {
    const int m = m0 + wm0 + 32 * i + lj;
    const bool row_ok = m < A.m;
    // int32 sums: the output (forward_acc, or inspection next to the bf16
    // output), or a K part's partial sums
    if (!bf || P.ksplit > 1 || (EPI && P.acc_out)) {
      const int ld = P.ksplit > 1 ? P.n : P.ldy;
      const bool wide = (ld & 3) == 0;  // rows are 16-byte aligned
      int32_t* yrow = (P.ksplit > 1 ? P.part + (int64_t)kp * A.m * P.n : P.acc_out) + (int64_t)m * ld;
#pragma unroll
      for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int n = n0 + wn0 + 32 * f + 8 * a + 4 * lg;
          if (!row_ok || n >= P.n) continue;
          const v4i v = {acc[i][f][4 * a], acc[i][f][4 * a + 1], acc[i][f][4 * a + 2], acc[i][f][4 * a + 3]};
          if (wide && n + 4 <= P.n) {
            *G(reinterpret_cast<v4i*>(yrow + n)) = v;
          } else {
            for (int e = 0; e < 4 && n + e < P.n; ++e) *G(yrow + n + e) = v[e];
          }
        }
      if constexpr (EPI) {
        if (!bf || P.ksplit > 1) continue;
      } else {
        continue;
      }
    }
    const RowDiv d = row_div_setup(xs[i] * ws);
    const bool wide = (P.ldy & 7) == 0;  // output rows are 16-byte aligned
    uint16_t* yrow = P.y + (int64_t)m * P.ldy;
#pragma unroll
    for (int f = 0; f < WNF; ++f) {
      float yf[16];
      if (d.fast) {
#pragma unroll
        for (int r = 0; r < 16; ++r) yf[r] = row_div_fast((float)acc[i][f][r], d.d, d.y);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) yf[r] = (float)acc[i][f][r] / d.d;
      }
      // pk[2a], pk[2a+1]: columns 8a + 4lg + 0..3 as bf16 pairs
      uint32_t pk[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) pk[h] = pack_bf16x2(yf[2 * h], yf[2 * h + 1]);
      // Swap lanes 32-63 of the first register with lanes 0-31 of the
      // second: lanes 0-31 then hold columns 0-7 (pk[0..3]) and 16-23
      // (pk[4..7]) of the 32-column subtile, lanes 32-63 columns 8-15 and
      // 24-31.
#pragma unroll
      for (int h = 0; h < 8; h += 4) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const auto sw = __builtin_amdgcn_permlane32_swap(pk[h + t], pk[h + 2 + t], false, false);
          pk[h + t] = sw[0];
          pk[h + 2 + t] = sw[1];
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + wn0 + 32 * f + 16 * h + 8 * lg;
        if (!row_ok || n >= P.n) continue;
        uint32_t w[4] = {pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
        if (wide && n + 8 <= P.n) {
          if constexpr (EPI) {
            if (P.bias) {
              const v4i b = *G(reinterpret_cast<const v4i*>(P.bias + n));
#pragma unroll
              for (int j = 0; j < 4; ++j) w[j] = add_bf16x2(w[j], (uint32_t)b[j]);
            }
            if (P.res) {
              const v4i r = *G(reinterpret_cast<const v4i*>(P.res + (int64_t)m * P.ldy + n));
#pragma unroll
              for (int j = 0; j < 4; ++j) w[j] = add_bf16x2(w[j], (uint32_t)r[j]);
            }
          }
          *G(reinterpret_cast<v4i*>(yrow + n)) = v4i{(int32_t)w[0], (int32_t)w[1], (int32_t)w[2], (int32_t)w[3]};
        } else {
          for (int e = 0; e < 8 && n + e < P.n; ++e) {
            uint16_t v = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            if constexpr (EPI) {
              if (P.bias) v = add_bf16(v, *G(P.bias + n + e));
              if (P.res) v = add_bf16(v, *G(P.res + (int64_t)m * P.ldy + n + e));
            }
            *G(yrow + n + e) = v;
          }
        }
      }
    }
  }
}

// Tiles are BNT = kPrefillBN columns wide, or kPrefillNarrowBN for the
// entries marked narrow: the host gives the tiles that would otherwise run
// in a last, partly filled round of workgroups that width, so that the
// round fills the chip and ends sooner.
// TBM: token rows per tile (the 32-row tiles take one 32-row subtile per
// wave, WMI = 1).
template <int NST, int WMI, int NW, int BK, bool EPI, int TBM>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW * kPrefillWgsPerCu / 4))) void prefill_kernel(const PrefillArgs A) {
  extern __shared__ __align__(16) int8_t smem[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i) pi += (i < A.count && (int)blockIdx.x >= A.tile_begin[i]);
  const PrefillProj& P = A.p[pi];
  int tm, tn;
  // the K parts of a split projection are further column tiles
  if (!tile_of((int)blockIdx.x - A.tile_begin[pi], A.tiles_m, P.tiles_n * P.ksplit, &tm, &tn)) return;
  const int kp = tn / P.tiles_n;
  tn -= kp * P.tiles_n;
  constexpr int W = TBM < 128 ? 1 : WMI;  // 32-row subtiles per wave
  if (P.narrow)
    prefill_tile<kPrefillNarrowBN, NST, W, NW, BK, EPI, TBM>(A, P, tm, tn, kp, smem);
  else
    prefill_tile<kPrefillBN, NST, W, NW, BK, EPI, TBM>(A, P, tm, tn, kp, smem);
}

// Adds the K parts of the split projections.  Piece i of a projection is 8
// consecutive outputs of one token row: the parts' int32 sums (part 0
// includes minus the row's code sum), then the same division and bf16
// rounding as the unsplit epilogue, or the int32 sum.
__global__ __launch_bounds__(kThreads) void prefill_finish_kernel(const PrefillArgs A) {
  const int idx = (int)blockIdx.x * kThreads + (int)threadIdx.x;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i) pi += (i < A.count && idx >= A.fin_begin[i]);
  const PrefillProj& P = A.p[pi];
  if (P.ksplit <= 1) return;
  const int cpr = (P.n + 7) >> 3;  // pieces per row
  const int local = idx - A.fin_begin[pi];
  if (local < 0 || local >= A.m * cpr) return;
  const int m = local / cpr, n = 8 * (local - m * cpr);
  const int64_t slice = (int64_t)A.m * P.n;
  const int32_t* src = P.part + (int64_t)m * P.n + n;
  const bool whole = n + 8 <= P.n;
  int32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if ((P.n & 3) == 0 && whole) {
    for (int kp = 0; kp < P.ksplit; ++kp) {
      const v4i lo = *G(reinterpret_cast<const v4i*>(src + kp * slice));
      const v4i hi = *G(reinterpret_cast<const v4i*>(src + kp * slice + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] += lo[e];
        v[4 + e] += hi[e];
      }
    }
  } else {
    for (int kp = 0; kp < P.ksplit; ++kp)
      for (int e = 0; e < 8 && n + e < P.n; ++e) v[e] += *G(src + kp * slice + e);
  }
  if (P.acc_out) {
    int32_t* dst = P.acc_out + (int64_t)m * P.ldy + n;
    if ((P.ldy & 3) == 0 && whole) {
      *G(reinterpret_cast<v4i*>(dst)) = v4i{v[0], v[1], v[2], v[3]};
      *G(reinterpret_cast<v4i*>(dst + 4)) = v4i{v[4], v[5], v[6], v[7]};
    } else {
      for (int e = 0; e < 8 && n + e < P.n; ++e) *G(dst + e) = v[e];
    }
  }
  if (!P.y) return;
  const RowDiv d = row_div_setup(*G(P.x_scale + m) * *G(P.w_scale));
  float yf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) yf[e] = d.fast ? row_div_fast((float)v[e], d.d, d.y) : (float)v[e] / d.d;
  uint16_t* dst = P.y + (int64_t)m * P.ldy + n;
  if ((P.ldy & 7) == 0 && whole) {
    uint32_t w[4] = {pack_bf16x2(yf[0], yf[1]), pack_bf16x2(yf[2], yf[3]),
                     pack_bf16x2(yf[4], yf[5]), pack_bf16x2(yf[6], yf[7])};
    if (P.bias) {
      const v4i b = *G(reinterpret_cast<const v4i*>(P.bias + n));
      for (int j = 0; j < 4; ++j) w[j] = add_bf16x2(w[j], (uint32_t)b[j]);
    }
    if (P.res) {
      const v4i r = *G(reinterpret_cast<const v4i*>(P.res + (int64_t)m * P.ldy + n));
      for (int j = 0; j < 4; ++j) w[j] = add_bf16x2(w[j], (uint32_t)r[j]);
    }
    *G(reinterpret_cast<v4i*>(dst)) = v4i{(int32_t)w[0], (int32_t)w[1], (int32_t)w[2], (int32_t)w[3]};
  } else {
    for (int e = 0; e < 8 && n + e < P.n; ++e) {
      uint16_t v = f32_to_bf16(yf[e]);
      if (P.bias) v = add_bf16(v, *G(P.bias + n + e));
      if (P.res) v = add_bf16(v, *G(P.res + (int64_t)m * P.ldy + n + e));
      *G(dst + e) = v;
    }
  }
}

// Slab buffers, wave layout and slab depth of the main variant: 4 waves of
// 64 x 128 outputs, slabs of 128 codes, two buffers of 24 KB -- small enough
// that two workgroups share a CU, so that one's epilogue (vector ALU work)
// overlaps the other's matrix-core loop.
#ifndef BL_PREFILL_NST
#define BL_PREFILL_NST 2
#endif
#ifndef BL_PREFILL_WMI
#define BL_PREFILL_WMI 2
#endif
#ifndef BL_PREFILL_NW
#define BL_PREFILL_NW 4
#endif
#ifndef BL_PREFILL_BK
#define BL_PREFILL_BK 128
#endif
static_assert(BL_PREFILL_BK == kPrefillSlab, "the host plans K parts in slabs of this size");

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int total_tiles, hipStream_t s) {
  if (a.load_mode == 0) {
    constexpr int BNT = BL_PREFILL_BN, NST = BL_PREFILL_NST, WMI = BL_PREFILL_WMI,
                  NW = BL_PREFILL_NW, BK = BL_PREFILL_BK;
    static_assert(BNT >= kPrefillNarrowBN, "the wide tiles' slab buffers hold the narrow ones'");
    bool ins = false;  // extra epilogue work: inspection, bias or residual
    for (int i = 0; i < a.count; ++i)
      ins = ins || (a.p[i].y && a.p[i].acc_out) || a.p[i].bias || a.p[i].res;
    auto go = [&](auto insc, auto bmc) -> hipError_t {
      constexpr bool I = decltype(insc)::value;
      constexpr int TB = decltype(bmc)::value;
      constexpr int W = TB < 128 ? 1 : WMI;
      // Small tiles do little work per slab, so more slabs stay in flight to
      // cover the memory latency (two workgroups per CU still fit the LDS).
      constexpr int NS = TB == 32 ? 6 : (TB == 64 ? 4 : NST);
      constexpr size_t lds = (size_t)NS * Cfg<BNT, W, NW, BK, TB>::kStageBytes;
      if (lds > 64 * 1024) {  // the attribute is needed above 64 KB; once per device
        static std::atomic<bool> done[kMaxDevices];
        const int dev = current_device_index();
        if (!done[dev].load(std::memory_order_acquire)) {
          const hipError_t attr = hipFuncSetAttribute(
              reinterpret_cast<const void*>(&prefill_kernel<NS, WMI, NW, BK, I, TB>),
              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (attr != hipSuccess) return attr;
          done[dev].store(true, std::memory_order_release);
        }
      }
      prefill_kernel<NS, WMI, NW, BK, I, TB><<<(unsigned)total_tiles, 64 * NW, lds, s>>>(a);
      return hipSuccess;
    };
    auto by_bm = [&](auto insc) -> hipError_t {
      if (a.bm == 32) return go(insc, std::integral_constant<int, 32>{});
      if (a.bm == 64) return go(insc, std::integral_constant<int, 64>{});
      return go(insc, std::integral_constant<int, kPrefillBM>{});
    };
    const hipError_t e = ins ? by_bm(std::true_type{}) : by_bm(std::false_type{});
    if (e != hipSuccess) return e;
  } else if (a.load_mode == 1) {
    prefill_reg_kernel<1><<<(unsigned)total_tiles, kThreads, 0, s>>>(a);
  } else {
    prefill_reg_kernel<2><<<(unsigned)total_tiles, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_finish(const PrefillArgs& a, int total_pieces, hipStream_t s) {
  if (total_pieces <= 0) return hipSuccess;
  prefill_finish_kernel<<<(unsigned)((total_pieces + kThreads - 1) / kThreads), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bl
