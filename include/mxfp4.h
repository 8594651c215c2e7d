/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 GEMM library, libmxfp4.so.
 *
 * The library computes C[M,N] = A[M,K] . B[N,K]^T with bf16 output, where A
 * arrives as bf16 and is quantized on the fly to MXFP4, and B arrives already
 * quantized.  MXFP4 here means: one e8m0 scale byte per 32 consecutive
 * K-elements of a row, and one 4-bit e2m1 code per element, two codes per
 * byte (element 2j in the low nibble of byte j).  Sources, all kernelindex.com
 * "kernelbot amd-mxfp4-mm" submissions:
 *   - scale rule: submission 752099 `_bf16_to_fp4_hw`, submission 754549
 *     `_quantize_mxfp4`, submission 739530 `hw_quant32` (zero group);
 *   - element rounding (nearest, ties to even, saturate at 6, sign on bit 3)
 *     and nibble order: submission 694791 `_mxfp4_quant_tile`;
 *   - block-scaled dot with fp32 accumulation: submission 752099
 *     `_quant_gemm_fused_launcher` (`tl.dot_scaled`), submission 739530
 *     `fgemm_pq` (the gfx950 scaled FP4 matrix instruction);
 *   - split-K with an fp32 workspace and a reduce pass: submission 739530
 *     `_gemm_k` / `_reduce_k`, submission 752099 `_splitk_sum_launcher`.
 *
 * Conventions for every call below:
 *   - pointers named a, b_*, c, workspace, *_packed and out_* are DEVICE
 *     pointers; the plan pointer is a HOST pointer;
 *   - `stream` is a hipStream_t (NULL = the default stream) of the current
 *     device, whose memory the device pointers must be; all device work is
 *     enqueued asynchronously on it and nothing is synchronised;
 *   - the library never allocates or frees device memory: the caller owns
 *     every buffer, and the size queries say how large each must be (the one
 *     exception, mxfp4_gemm_noalloc, uses a fixed array inside the library
 *     instead of a caller's workspace);
 *   - an empty call -- M = 0 for the quantizers, N = 0 for mxfp4_pack_b,
 *     M = 0 or N = 0 for the GEMMs, with K still a positive multiple of 32
 *     -- returns 0 and enqueues nothing; its pointers and other arguments
 *     are not read (they may be NULL).  The size queries give 0 for it;
 *     mxfp4_default_plan and mxfp4_check_plan refuse it (an empty product
 *     has no plan);
 *   - return value 0 is success; a negative value is one of MXFP4_E* below.
 *     On any error other than MXFP4_EHIP nothing has been enqueued.  The
 *     text of the last error of the calling thread is mxfp4_last_error();
 *   - calls are thread-safe; apart from mxfp4_gemm_noalloc's per-GPU
 *     scratch array the library holds no device state between calls;
 *   - a call enqueues kernel launches only (no allocation, memset or
 *     synchronization), so it can be captured into a HIP graph; a replay
 *     reads the buffers as they are at replay time, and replays that share
 *     a workspace must not overlap, like calls.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP4_OK 0
#define MXFP4_EINVAL (-1)     /* bad shape, stride or alignment */
#define MXFP4_ENULL (-2)      /* a required pointer is NULL */
#define MXFP4_EWORKSPACE (-3) /* workspace smaller than the plan needs */
#define MXFP4_ESIZE (-4)      /* a packed buffer is smaller than its layout */
#define MXFP4_ENOTSUP (-5)    /* plan fields with no compiled kernel */
#define MXFP4_EHIP (-6)       /* the HIP runtime reported a launch error */

/* ------------------------------------------------------------------------
 * Packed operand layout ("MX-packed").
 *
 * Both the pre-packed B and the pre-quantized A use one layout, laid out in
 * the lane order of the gfx950 block-scaled 16x16x128 FP4 matrix instruction
 * (lane L holds row L%16 and the 32-element K-group L/16 of a 128-K step).
 * For a matrix of R rows and K columns (K % 32 == 0; K is padded up to whole
 * 128-element steps):
 *     RT = ceil(R/16) row tiles, KS = ceil(K/128) steps, KG = ceil(KS/4),
 *     data bytes  D = RT*KS*1024,  total bytes = D + RT*KG*256.
 *   data:  byte ((t*KS + j)*64 + L)*16 + i  holds linear fp4x2 byte
 *          (64*j + 16*(L/16) + i) of row 16*t + L%16,  i in [0,16);
 *   scale: byte D + ((t*KG + g)*64 + L)*4 + s  holds the e8m0 scale of row
 *          16*t + L%16, K-group 4*(4*g + s) + L/16, for step 4*g+s < KS;
 *          bytes for steps >= KS hold 127.
 * Padding -- rows >= R, and K-groups at or beyond K/32 -- holds code 0 and
 * scale 127 (a zero contribution to any product).
 * ---------------------------------------------------------------------- */

/* Bytes of the MX-packed layout for `rows` rows of K columns; 0 when
 * rows < 1 or K is not a positive multiple of 32. */
size_t mxfp4_packed_bytes(int rows, int K);

/* One-time repack of a quantized B into the MX-packed layout.
 * The pages receive B already quantized and pre-shuffled for the matrix
 * instruction and never time that step (submission 752099, the harness's
 * `B_shuffle` / `B_scale_sh` operands); submission 739530 `fgemm_pq` shows
 * what the instruction needs per lane: 16 bytes of codes of one row's
 * 32-element K-group and that group's scale byte.  This call is that
 * one-time step for this library's own layout.
 *   b_fp4   [N][K/2]  fp4x2, row-major, contiguous (16-byte aligned);
 *   b_scale [N][K/32] e8m0,  row-major, contiguous;
 *   b_packed  output, mxfp4_packed_bytes(N, K) bytes, 16-byte aligned.
 * Requires N >= 0 (0: an empty call), K >= 32, K % 32 == 0.  This is a byte permutation only
 * (no arithmetic).  Errors: ENULL, EINVAL, ESIZE, EHIP. */
int mxfp4_pack_b(const uint8_t *b_fp4, const uint8_t *b_scale, int N, int K, void *b_packed,
                 size_t b_packed_bytes, void *stream);

/* Quantize bf16 rows to MXFP4 in the linear layout.
 *   a        [M][lda] bf16 bit patterns (uint16), 16-byte aligned, lda % 8 == 0;
 *   out_fp4  [M][ld_fp4] bytes, row m gets K/2 bytes, ld_fp4 >= K/2, ld_fp4 % 4 == 0,
 *            4-byte aligned;
 *   out_scale [M][ld_scale] bytes, row m gets K/32 bytes, ld_scale >= K/32.
 * Requires M >= 0 (0: an empty call), K >= 32, K % 32 == 0, lda >= K.  The group scale is the
 * rule of submission 752099 `_bf16_to_fp4_hw`; elements round to nearest
 * e2m1 with ties to even and saturate at 6 (submission 694791).  Results are
 * bit-exact to that definition.  Errors: ENULL, EINVAL, EHIP. */
int mxfp4_quant_a(const uint16_t *a, int M, int K, int lda, uint8_t *out_fp4, int ld_fp4,
                  uint8_t *out_scale, int ld_scale, void *stream);

/* Quantize bf16 rows straight into the MX-packed layout (the layout the
 * GEMM reads), padding rows included.  The separate pre-quantization of A
 * of submission 739530 (`prequant`: codes and scales written once, then
 * read by the GEMM), with the scale and element rules of mxfp4_quant_a,
 * written in the GEMM's operand layout instead of a linear one.
 *   a  as for mxfp4_quant_a;  out_packed  mxfp4_packed_bytes(M, K) bytes,
 *   16-byte aligned.  Requires M >= 0 (0: an empty call), K >= 32, K % 32 == 0.  Applied to a
 *   weight matrix B [N][K] this is the one-time B preparation straight from
 *   bf16 (the same bytes as mxfp4_quant_a followed by mxfp4_pack_b).
 *   Errors: ENULL, EINVAL, ESIZE, EHIP. */
int mxfp4_quant_a_packed(const uint16_t *a, int M, int K, int lda, void *out_packed,
                         size_t out_packed_bytes, void *stream);

/* ------------------------------------------------------------------------
 * GEMM plans.
 *
 * A plan fixes how one call is split over the GPU.  The work is
 * ceil(ceil(M/16)/m_blocks) row groups times
 * ceil((N/16)/(waves_n*n_tiles_per_wave)) * split_k column tasks, one
 * workgroup of waves_n*waves_k wavefronts each (the row groups of one column
 * task are placed on one XCD); each wavefront owns
 * n_tiles_per_wave 16-column tiles of B, m_blocks 16-row blocks of A, and
 * k_steps_per_wave 128-element K-steps.  The K steps must be covered
 * exactly: split_k * waves_k * k_steps_per_wave == ceil(K/128).  waves_k > 1 sums
 * the wavefronts' partial tiles in LDS (fixed order); split_k > 1 writes fp32
 * partials [split_k][M][N] to the workspace and sums them in order
 * s = 0..split_k-1, rounding to bf16 (nearest even) -- either in a separate
 * reduce kernel (split_reduce = MXFP4_REDUCE_KERNEL) or, in the same launch,
 * in the last workgroup to finish each output tile, found with a per-tile
 * arrival counter in the workspace (MXFP4_REDUCE_LAST_WG).  Both give the
 * same bits.  MXFP4_REDUCE_ATOMIC instead adds every slice's fp32 partial
 * into one [M][N] accumulator in the workspace with atomic adds, and the last
 * workgroup of each tile rounds the sum to bf16 and clears the accumulator;
 * the order of the additions varies from call to call, so its results agree
 * with the others within the fp32 rounding of a different summation order,
 * not bit for bit.
 *
 * mode FUSED quantizes the workgroup's A rows inside the GEMM kernel; mode
 * PREQUANT first runs the quantizer once into the workspace (MX-packed) and
 * the GEMM kernel reads fp4 A.
 *
 * mode TILED is the large-M kernel: like PREQUANT it quantizes A into the
 * workspace first, then one workgroup computes each tile of C over the
 * whole of K with the gfx950 block-scaled 32x32x64 FP4 instruction (the
 * same products and fp32 sums per output as the other modes, in K order;
 * results agree with them within fp32 rounding, not bit for bit).
 * waves_n == 2 selects 256 x 128 tiles, any other value 256 x 256 tiles
 * (eight wavefronts either way); both widths give the same bits.  split_k
 * > 1 shares each tile's K among split_k workgroups of
 * 4*ceil(ceil(ceil(K/128)/split_k)/4) steps each (none may be left empty:
 * split_k <= ceil(ceil(K/128)/4) and (split_k-1) times that < ceil(K/128)),
 * whose fp32 partials [split_k][M][N] in the workspace the reduce kernel
 * sums in order (split_reduce must be MXFP4_REDUCE_KERNEL).  The other
 * fields are not read.  K must be <= 4194304 (2^22).  It pays off when M
 * and N give many tiles, or, split, when K is long.
 *
 * mode STREAM is the K-looping kernel for small and mid M: like PREQUANT it quantizes
 * A into the workspace first; then each workgroup of four wavefronts (one
 * group of n_tiles_per_wave 16-column tiles each) takes m_blocks 16-row
 * blocks of A over a range of k_steps_per_wave 128-K steps (a multiple of
 * 4, up to ceil(K/128) rounded up to 4), looping over it four steps at a
 * time (A through LDS, B straight into registers), and split_k =
 * ceil(ceil(ceil(K/128)/4) / (k_steps_per_wave/4)) workgroups cover K,
 * their fp32 partials summed by the reduce kernel (split_reduce must be
 * MXFP4_REDUCE_KERNEL).  waves_n must be 4 and waves_k 1.  Same products
 * as the other modes with the 16x16x128 instruction; the sums differ only
 * in order.  K must be <= 4194304 (2^22).
 * ---------------------------------------------------------------------- */
#define MXFP4_MODE_FUSED 1
#define MXFP4_MODE_PREQUANT 2
#define MXFP4_MODE_TILED 3
#define MXFP4_MODE_STREAM 4

#define MXFP4_REDUCE_KERNEL 0
#define MXFP4_REDUCE_LAST_WG 1
#define MXFP4_REDUCE_ATOMIC 2

typedef struct mxfp4_plan {
    int mode;             /* MXFP4_MODE_FUSED, _PREQUANT, _TILED or _STREAM */
    int m_blocks;         /* 16-row blocks of A per workgroup: 1, 2 or 4 */
    int n_tiles_per_wave; /* 16-column tiles of B per wavefront: 1 or 2 */
    int waves_n;          /* wavefronts along N per workgroup */
    int waves_k;          /* wavefronts along K per workgroup (in-LDS reduce);
                             waves_n * waves_k <= 8 */
    int k_steps_per_wave; /* 128-K steps per wavefront: 1,2,3,4,6,7,8,12,14,16 */
    int split_k;          /* workgroups along K (fp32 workspace + reduce) */
    int split_reduce;     /* split_k > 1: MXFP4_REDUCE_KERNEL, MXFP4_REDUCE_LAST_WG
                             (needs split_k <= 16) or MXFP4_REDUCE_ATOMIC */
} mxfp4_plan;

/* The plan mxfp4_gemm uses for a shape: a per-shape table for the tuned
 * shapes; for M up to 512 against a B with K >= 4096, the stream mode or a
 * fused plan that splits K, where measured rules take them; otherwise the
 * plan of least estimated time under a cost model (fused, pre-quantized or,
 * when M >= 256 and M and N give at least 16 tiles of 256 x 256, tiled with
 * either tile width and K split over up to eight workgroups).  A tiled
 * plan's fields other than mode, waves_n, split_k and split_reduce are 1
 * and unused.
 * Errors: ENULL, EINVAL (also for an empty shape). */
int mxfp4_default_plan(int M, int N, int K, mxfp4_plan *plan);

/* MXFP4_OK when `plan` is valid for the shape and has a compiled kernel;
 * otherwise the status mxfp4_gemm_ex would return for it (EINVAL, ENOTSUP,
 * ENULL), with the reason in mxfp4_last_error(). */
int mxfp4_check_plan(const mxfp4_plan *plan, int M, int N, int K);

/* Workspace bytes a plan needs for a shape, laid out as
 *   [tile counters][fp32 partials or accumulator][MX-packed A]
 * with each part rounded up to 256 bytes: tile counters (4 bytes per
 * workgroup tile) when split_k > 1 and split_reduce is LAST_WG or ATOMIC;
 * split_k*M*N*4 bytes of partials when split_k > 1 (M*N*4 bytes, one
 * accumulator, for ATOMIC); the MX-packed A in PREQUANT and TILED mode
 * (TILED needs nothing else).
 * 0 when none is needed or the plan is invalid. */
size_t mxfp4_plan_workspace_bytes(const mxfp4_plan *plan, int M, int N, int K);

/* Leading workspace bytes (the tile counters, and for ATOMIC the
 * accumulator after them) that must be zero before the first call that uses
 * the workspace with this plan; every completed call leaves them zero again,
 * so one zero-fill per workspace suffices.  Calls that share one workspace
 * must not overlap in time.  The rest of the workspace is scratch.  0 when
 * the plan keeps no counters. */
size_t mxfp4_plan_workspace_zero_bytes(const mxfp4_plan *plan, int M, int N, int K);

/* Workspace bytes of the default plan (same layout and zero-fill rule). */
size_t mxfp4_gemm_workspace_bytes(int M, int N, int K);

/* C = A . B^T with the default plan: the block-scaled product of
 * submission 752099 `_quant_gemm_fused_launcher` (A quantized in the
 * kernel, `tl.dot_scaled` of two e2m1 operands with their e8m0 scales,
 * fp32 accumulation, bf16 result) and submission 739530 `fgemm_pq` (the
 * gfx950 scaled FP4 matrix instruction; rows past M take scale 0 and are
 * not stored).  C[m][n] = sum over k of deqA[m][k] * deqB[n][k], summed in
 * fp32 in an order that depends on the plan, rounded to bf16 (nearest even).
 *   a         [M][lda] bf16, 16-byte aligned, lda % 8 == 0, lda >= K;
 *   b_packed  MX-packed B of N rows (from mxfp4_pack_b), b_packed_bytes >=
 *             mxfp4_packed_bytes(N, K);
 *   c         [M][ldc] bf16 output, ldc >= N; only the M x N block is written;
 *   workspace device scratch of at least mxfp4_gemm_workspace_bytes(M,N,K)
 *             bytes, 256-byte aligned (may be NULL when that is 0), whose
 *             leading zero-bytes (see mxfp4_plan_workspace_zero_bytes) were
 *             zero-filled once before first use.
 * Requires M >= 0, N >= 0 (either 0: an empty call), K >= 32, K % 32 == 0.
 * Inputs are finite.  c must not overlap a, b_packed or the workspace (the
 * kernels read the inputs while other workgroups already write C).
 * Errors: ENULL, EINVAL, ESIZE, EWORKSPACE, ENOTSUP, EHIP. */
int mxfp4_gemm(const uint16_t *a, int lda, const void *b_packed, size_t b_packed_bytes,
               uint16_t *c, int ldc, int M, int N, int K, void *workspace,
               size_t workspace_bytes, void *stream);

/* As mxfp4_gemm with an explicit plan (NULL = default plan).  The plan
 * chooses among the pages' schemes: A quantized inside the GEMM (submission
 * 752099 `_quant_gemm_fused_launcher`) or by a separate pre-quantization
 * launch (submission 739530 `prequant` + `fgemm_pq`), and K split over
 * workgroups with fp32 partials summed by a second kernel (submission 752099
 * `_splitk_sum_launcher`, submission 739530 `_reduce_k`). */
int mxfp4_gemm_ex(const uint16_t *a, int lda, const void *b_packed, size_t b_packed_bytes,
                  uint16_t *c, int ldc, int M, int N, int K, void *workspace,
                  size_t workspace_bytes, const mxfp4_plan *plan, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): C = A . B^T
 * with the default plan, as mxfp4_gemm, but with no workspace argument.  The
 * scratch the plan needs (split-K partials, the pre-quantized A) lives in a
 * fixed array inside the library, one copy per GPU, of
 * mxfp4_gemm_noalloc_max_scratch_bytes() bytes (16 MiB), held from the
 * library's first use of that GPU until the process ends; the call allocates
 * and frees nothing.  Shapes whose default plan needs more scratch than that
 * (mxfp4_gemm_workspace_bytes) are refused with MXFP4_EWORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array and
 * the array keeps the last call's contents (parts that must start at zero
 * are cleared by the call itself, with a fill kernel): calls on one GPU
 * that may overlap in time -- on different streams, or from several threads
 * without ordering -- race on it and give undefined results; serialize
 * them, or use mxfp4_gemm with one workspace per stream.  Results are those
 * of mxfp4_gemm bit for bit.  The first call on a GPU looks up that GPU's
 * copy of the array (hipGetSymbolAddress); make that call outside a HIP
 * graph capture: every later call enqueues kernel launches only, so it can
 * be captured like mxfp4_gemm.
 * Arguments and errors: as mxfp4_gemm, plus EWORKSPACE for too large a
 * shape. */
int mxfp4_gemm_noalloc(const uint16_t *a, int lda, const void *b_packed, size_t b_packed_bytes,
                       uint16_t *c, int ldc, int M, int N, int K, void *stream);

/* Bytes of the per-GPU scratch array of mxfp4_gemm_noalloc. */
size_t mxfp4_gemm_noalloc_max_scratch_bytes(void);

/* Workspace bytes of mxfp4_gemm_prequant for a plan (NULL = default plan);
 * its zero-fill prefix is mxfp4_plan_workspace_zero_bytes of the same plan. */
size_t mxfp4_gemm_prequant_workspace_bytes(const mxfp4_plan *plan, int M, int N, int K);

/* GEMM on an A that is already MX-packed (from mxfp4_quant_a_packed), for
 * callers that quantize one activation once and use it against several
 * weights: the GEMM half of submission 739530's two-kernel path
 * (`fgemm_pq`, A read as fp4 codes and scale bytes).  Plan mode
 * MXFP4_MODE_TILED runs the tiled kernel (no workspace);
 * any other mode value means the plan's tiling with fp4 A, as in PREQUANT
 * mode.  NULL plan = the default plan.  Workspace: as for mxfp4_gemm_ex with
 * the plan in PREQUANT mode, minus the MX-packed A part (tile counters, then
 * partials).
 * Errors: ENULL, EINVAL, ESIZE, EWORKSPACE, ENOTSUP, EHIP. */
int mxfp4_gemm_prequant(const void *a_packed, size_t a_packed_bytes, const void *b_packed,
                        size_t b_packed_bytes, uint16_t *c, int ldc, int M, int N, int K,
                        void *workspace, size_t workspace_bytes, const mxfp4_plan *plan,
                        void *stream);

/* Text of the last error returned on the calling thread ("" if none). */
const char *mxfp4_last_error(void);

/* Library version string. */
const char *mxfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
