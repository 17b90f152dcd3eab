/*
 * bitlinear.h -- C ABI of libbitlinear.so, the BitNet b1.58 BitLinear forward
 * pass on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: the Falcon-Edge blog, rendered in Arabic on
 * n77n.net as "A series of powerful, universal and fine-tunable 1.58-bit
 * language models", section "Falcon-Edge, a series of universal models",
 * functions activation_norm_quant, _weight_quant, BitLinear.forward and
 * BitLinear.post_quant_process; and the GeekNews page "BitNet: an inference
 * framework for 1-bit LLMs", section "Hacker News comments", on 2-bit
 * storage):
 *
 *   weights   : w_scale = 1 / max(mean|w|, 1e-5)            (per tensor)
 *               u = clamp(round(w * w_scale), -1, 1)        (ternary)
 *   activations: x_scale[m] = 127 / max(max_k |x[m,k]|, 1e-5) (per token)
 *               q = clamp(round(x * x_scale), -128, 127)    (int8)
 *   contraction: acc[m,n] = sum_k q[m,k] * u[n,k]          (exact int32)
 *   output    : y[m,n] = bf16(acc[m,n] / (x_scale[m] * w_scale))
 *
 * Arithmetic: IEEE fp32, round-to-nearest-even for the multiplies, the
 * correctly rounded divisions and round(); 1e-5 is fp32(1e-5); mean|w| is
 * the exact sum of |w| over the element count, rounded once to fp32 (so it
 * does not depend on summation order); the output is rounded to bf16 with
 * round-to-nearest-even.  Every result is deterministic and bit-identical
 * from run to run.
 *
 * Packed weight format: row-major [N][K/4] bytes.  Byte k/4 of row n holds
 * weight k at bits 2*(k%4)..2*(k%4)+1 as the code c = u + 1 (0, 1 or 2).
 * Code 3 is never written; if present in caller data it decodes as +2.
 *
 * Tiled weight layout (optional, N % 16 == 0 and K % 256 == 0): the same
 * N*K/4 bytes, permuted inside every block of 16 rows.  The block of rows
 * 16b..16b+15 keeps its place (bytes 16b*K/4 .. (16b+16)*K/4) and is stored
 * as K/256 tiles of 1 KB, tile t holding packed bytes 64t..64t+63 of each of
 * its 16 rows: the 16-byte chunk g (0..3) of row 16b+r sits at byte
 * 1024t + 256g + 16r of the block.  Row-major byte o of row n is therefore
 * at (n/16)*16*(K/4) + 1024*(o/64) + 256*((o/16)%4) + 16*(n%16) + o%16.
 * Each tile is what one 64-lane wavefront reads for a 16-row operand of the
 * 16x16x64 int8 matrix-core op, so decode streams the weights in contiguous
 * 1 KB pieces.  bitlinear_tile_weights / bitlinear_untile_weights convert;
 * the *_tiled entry points and bl_projection.layout take it.  Results are
 * identical to those on the row-major bytes.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major data,
 *    owned by the caller.  The library never allocates, frees, or
 *    synchronizes, and keeps no state between calls apart from per-device
 *    facts it looks up once (the CU count, kernel LDS limits, and the device
 *    address of the no-alloc entry point's scratch array); calls are
 *    thread-safe, except that no-alloc calls on one GPU must not overlap.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued; results are ready once the stream has reached that point.
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    any error nothing is enqueued and the status says why.  A failed
 *    launch returns BL_EHIP.  Faults inside kernels surface at the caller's
 *    next synchronization, as with any HIP work.
 *  - Shapes: M, N, K >= 1; K % 4 == 0; K <= 2^22; N <= 2^30; M <= 2^24;
 *    M*K, N*K/4 and M*N each below 2^40.
 *  - Alignment: every pointer 16-byte aligned (what hipMalloc and the
 *    PyTorch caching allocator return for a tensor's storage).
 *  - Inputs must be finite; non-finite inputs give unspecified outputs.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BL_OK = 0,
  BL_EINVAL = 1,     /* null pointer, or count/argument out of range */
  BL_ESHAPE = 2,     /* M, N or K out of the supported range, K % 4 != 0 */
  BL_EALIGN = 3,     /* a pointer is not 16-byte aligned */
  BL_EWORKSPACE = 4, /* workspace pointer null or smaller than required */
  BL_EHIP = 5        /* a kernel launch failed */
} bl_status;

/* One projection of a grouped forward call (host-side descriptor).
 * Optional epilogue (BitLinear.forward's bias line, and the residual add of
 * the block around the layer): the bf16 output of the dequantization gets
 * bias[n] added, then residual[m][n]; each add is one fp32 addition of the
 * two bf16 values rounded to bf16 (round to nearest even), as a bf16 tensor
 * add.  NULL skips the step. */
typedef struct {
  const uint16_t *x;        /* [M][K] bf16 activations (device) */
  const uint8_t *packed;    /* [N][K/4] packed ternary weights (device) */
  const float *w_scale;     /* 1 float, the weight scale (device) */
  uint16_t *y;              /* [M][N] bf16 output (device) */
  int64_t n;                /* N, output features */
  int64_t k;                /* K, input features */
  int32_t layout;           /* BL_LAYOUT_ROWS (0) or BL_LAYOUT_TILED (1) */
  int32_t reserved;         /* must be 0 */
  const uint16_t *bias;     /* [N] bf16 bias (device, 16-byte aligned), or NULL */
  const uint16_t *residual; /* [M][N] bf16 (device, 16-byte aligned), or NULL; may be
                               y itself (an in-place residual add), must not
                               otherwise overlap y */
} bl_projection;

/* Weight layouts (bl_projection.layout). */
#define BL_LAYOUT_ROWS 0  /* row-major [N][K/4] */
#define BL_LAYOUT_TILED 1 /* 16-row tiled (N % 16 == 0, K % 256 == 0) */

/* Human-readable name of a status code (static string, never NULL). */
const char *bitlinear_status_string(bl_status s);

/* Interface version of this header; bumped on any ABI change. */
int bitlinear_abi_version(void);

/* --- weight preparation (offline) ------------------------------------- */

/* Bytes of workspace bitlinear_pack_weights needs (independent of sizes:
 * 256 64-bit exponent buckets). */
size_t bitlinear_pack_workspace_bytes(int64_t n, int64_t k);

/* Ternarize and pack latent weights: the blog's _weight_quant followed by
 * 2-bit storage.  w: [N][K] fp32.  packed: [N][K/4] bytes (written).
 * w_scale: 1 float (written) = 1 / max(mean|w|, 1e-5).  The mean is exact
 * (order independent).  workspace: at least
 * bitlinear_pack_workspace_bytes(n, k) bytes of device memory; its contents
 * on entry do not matter and are clobbered.  Enqueues four kernels. */
bl_status bitlinear_pack_weights(const float *w, int64_t n, int64_t k,
                                 uint8_t *packed, float *w_scale,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/* The "universal" bf16 export (the blog's state_dict loop after
 * _weight_quant): out[n][k] = bf16(u[n][k] / w_scale), one correctly rounded
 * fp32 division rounded to bf16, from packed weights in either layout
 * (layout: BL_LAYOUT_ROWS or BL_LAYOUT_TILED; tiled needs N % 16 == 0 and
 * K % 256 == 0).  out: [N][K] bf16, row-major (written).  One kernel. */
bl_status bitlinear_export_bf16(const uint8_t *packed, int64_t n, int64_t k,
                                int32_t layout, const float *w_scale,
                                uint16_t *out, void *stream);

/* Expand packed weights to int8 values c - 1: [N][K/4] -> [N][K].
 * (The blog's unpack_weights; used to inspect stored weights.) */
bl_status bitlinear_unpack_weights(const uint8_t *packed, int64_t n,
                                   int64_t k, int8_t *u, void *stream);

/* Row-major packed weights -> the tiled layout (a byte permutation; see
 * above).  packed: [N][K/4]; tiled: N*K/4 bytes (written).  N % 16 == 0 and
 * K % 256 == 0, else BL_ESHAPE; the two arrays must not overlap (BL_EINVAL).
 * One kernel. */
bl_status bitlinear_tile_weights(const uint8_t *packed, int64_t n, int64_t k,
                                 uint8_t *tiled, void *stream);

/* The inverse: tiled layout -> row-major [N][K/4].  Same rules. */
bl_status bitlinear_untile_weights(const uint8_t *tiled, int64_t n, int64_t k,
                                   uint8_t *packed, void *stream);

/* --- activation quantization ------------------------------------------ */

/* The blog's activation_norm_quant on bf16 input.  x: [M][K] bf16.
 * q: [M][K] int8 (written).  x_scale: [M] fp32 (written). */
bl_status bitlinear_act_quant(const uint16_t *x, int64_t m, int64_t k,
                              int8_t *q, float *x_scale, void *stream);

/* --- forward ----------------------------------------------------------- */

/* Bytes of workspace bitlinear_forward needs for this shape. */
size_t bitlinear_forward_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* BitLinear.forward without bias: y = bf16(q(x) . u^T / (x_scale*w_scale)).
 * x: [M][K] bf16; packed: [N][K/4]; w_scale: 1 float (device); y: [M][N]
 * bf16 (written).  workspace: at least
 * bitlinear_forward_workspace_bytes(m, n, k) bytes; contents on entry do
 * not matter.  M <= 16 runs the decode GEMV path, larger M the int8
 * matrix-core GEMM path; both give identical results.  Enqueues one to
 * three kernels, by M, K and the launch plan: the decode kernel alone when
 * it quantizes the activations itself; otherwise an activation-quantization
 * kernel, then the contraction, and for a GEMM whose K is split across
 * workgroups a pass that adds the parts. */
bl_status bitlinear_forward(int64_t m, int64_t n, int64_t k,
                            const uint16_t *x, const uint8_t *packed,
                            const float *w_scale, uint16_t *y,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/* Bytes of workspace bitlinear_forward_latent needs for this shape. */
size_t bitlinear_forward_latent_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* The forward pass on latent fp32 weights, ternarized on the fly (the
 * blog's two-stage approach for its training kernels: a global reduction
 * first, then block-wise quantization): the exact absmean of w [N][K] fp32,
 * then ternarization and packing into the workspace, then
 * bitlinear_forward on them.  Results are identical to
 * bitlinear_pack_weights followed by bitlinear_forward.  w_scale: 1 float
 * (device, written) or NULL (kept in the workspace).  workspace: at least
 * bitlinear_forward_latent_workspace_bytes(m, n, k) bytes.  Enqueues the
 * four packing kernels, then the forward's. */
bl_status bitlinear_forward_latent(int64_t m, int64_t n, int64_t k,
                                   const uint16_t *x, const float *w,
                                   float *w_scale, uint16_t *y, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* bitlinear_forward with the weights in the tiled layout (N % 16 == 0,
 * K % 256 == 0, else BL_ESHAPE).  Workspace:
 * bitlinear_forward_workspace_bytes(m, n, k).  Same results. */
bl_status bitlinear_forward_tiled(int64_t m, int64_t n, int64_t k,
                                  const uint16_t *x, const uint8_t *tiled,
                                  const float *w_scale, uint16_t *y,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Bytes of workspace bitlinear_forward_grouped needs (the layouts do not
 * change it). */
size_t bitlinear_forward_grouped_workspace_bytes(int32_t count,
                                                 const bl_projection *projs,
                                                 int64_t m);

/* Kernels one bitlinear_forward_grouped call with these shapes enqueues (1
 * to 3: see bitlinear_forward), or -1 for invalid arguments.  Host only;
 * only the shapes of `projs` are read. */
int32_t bitlinear_forward_grouped_launches(int32_t count, const bl_projection *projs,
                                           int64_t m);

/* Several independent BitLinear forwards with the same token count M (for
 * instance the projections of one decoder layer) in one pass: at most one
 * activation-quantization launch, one contraction launch and one pass that
 * adds K parts, for all of them together.  projs: HOST array of `count` descriptors (1 <= count <= 16);
 * results are identical to calling bitlinear_forward on each.  Each
 * descriptor names its weights' layout; an unknown layout is BL_EINVAL, a
 * tiled one with N % 16 != 0 or K % 256 != 0 is BL_ESHAPE. */
bl_status bitlinear_forward_grouped(int32_t count, const bl_projection *projs,
                                    int64_t m, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Side outputs of a forward call, for inspecting the values the forward
 * path itself computed (all DEVICE pointers, 16-byte aligned; each may be
 * NULL, and is then not written). */
typedef struct {
  int8_t *q;        /* [M][K] the int8 codes x was quantized to (the blog's
                       activation_norm_quant), natural row-major layout */
  float *x_scale;   /* [M] the per-token scales 127 / max(max_k |x|, 1e-5) */
  int32_t *qsum;    /* [M] sum over k of q[m][k] */
  int32_t *acc;     /* [M][N] the exact accumulators sum_k q[m][k] * u[n][k] */
} bl_inspect;

/* bitlinear_forward_grouped with inspection: the same plans, kernels and
 * outputs y, and in addition the codes, scales, code sums and int32
 * accumulators each projection's kernels computed (inspect: HOST array of
 * `count` bl_inspect).  wait_polls bounds the waits between the waves of a
 * decode workgroup (0: the default, 2^24 polls; negative: every such wait
 * gives up at once, which exercises the error report).  A workgroup whose
 * wait gave up writes NaN (bf16 0x7FC0) outputs and INT32_MIN accumulators,
 * and if `status` (a DEVICE int32, may be NULL) is given ORs 1 into it; the
 * library never clears it.  The other entry points use the default bound
 * and no status word (their outputs are still poisoned on a give-up). */
bl_status bitlinear_forward_grouped_inspect(int32_t count, const bl_projection *projs,
                                            int64_t m, const bl_inspect *inspect,
                                            int32_t *status, int32_t wait_polls,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * bitlinear_forward_grouped without a workspace argument.  Its scratch
 * memory is a fixed array of BL_NOALLOC_SCRATCH_BYTES in the library's code
 * object; each GPU the library runs on holds its own copy until the process
 * ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); on its first use on a device it looks up that device's
 * copy of the array.  Arguments, results and launches are those of
 * bitlinear_forward_grouped; a call whose
 * bitlinear_forward_grouped_workspace_bytes exceeds BL_NOALLOC_SCRATCH_BYTES
 * returns BL_EWORKSPACE and enqueues nothing.  Every call on one GPU uses the
 * same array (the library clears what must start at zero): calls that
 * overlap on one GPU -- on different streams, or from different threads --
 * race and give undefined results; serialize them. */
#define BL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
bl_status bitlinear_forward_grouped_noalloc(int32_t count, const bl_projection *projs,
                                            int64_t m, void *stream);

/* Integer accumulators of caller-supplied int8 codes: acc = q . u^T.
 * q: [M][K] int8 (any values); packed: [N][K/4]; acc: [M][N] int32
 * (written).  Runs the same contraction kernels as bitlinear_forward (the
 * path chosen by M) with an int32 epilogue; exposes the exact accumulators
 * for inspection.  workspace: bitlinear_forward_workspace_bytes(m, n, k). */
bl_status bitlinear_forward_acc(int64_t m, int64_t n, int64_t k,
                                const int8_t *q, const uint8_t *packed,
                                int32_t *acc, void *workspace,
                                size_t workspace_bytes, void *stream);

/* bitlinear_forward_acc with the weights in the tiled layout (N % 16 == 0,
 * K % 256 == 0, else BL_ESHAPE). */
bl_status bitlinear_forward_acc_tiled(int64_t m, int64_t n, int64_t k,
                                      const int8_t *q, const uint8_t *tiled,
                                      int32_t *acc, void *workspace,
                                      size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
