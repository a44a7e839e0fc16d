/*
 * libmxgemm — MXFP4 block-scaled GEMM for AMD Instinct MI355X (gfx950).
 *
 *     D[M,N] = bf16( alpha * A[M,K] * B[N,K]^T + beta * C[M,N] )
 *
 * A and B hold OCP E2M1 (fp4) codes packed two per byte; every run of 32
 * consecutive K elements of a row carries one E8M0 scale byte.  This is the
 * problem the asm_f4gemm README ("asm_f4gemm -- driving aiter's gfx950
 * MXFP4 GEMM code objects") states at its top; operand formats follow its
 * section "Data layouts":
 *
 *   A      [M][lda/2] bytes, row-major.  Byte i of a row holds element 2i in
 *          its low nibble and element 2i+1 in its high nibble.  A code's
 *          value is one of {0, .5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
 *   B      [N][ldb/2] bytes, same encoding (B is used transposed: D = A B^T).
 *   scaleA [M][ldsa] bytes: scaleA[i][k/32] is the E8M0 scale of A[i][k];
 *          its value is 2^(e-127) (0xFF is NaN).
 *   scaleB [N][ldsb] bytes, likewise for B.
 *   C, D   [M][ldc], [M][ldd] bf16, row-major.
 *
 * Arithmetic: the scaled products are accumulated in fp32 by the CDNA4
 * scaled matrix instructions ("CDNA4 dense MFMA builtins", section
 * "Mixed-precision with scaling"), partial sums of a split K are added in
 * fp32 in a fixed order, and the epilogue forms alpha*acc + beta*C in fp32
 * and rounds once to bf16 (nearest, ties to even).  When beta == 0, C is not
 * read (it may be NULL and may hold NaNs).
 *
 * Every pointer passed to libmxgemm is a DEVICE pointer on the current HIP
 * device, owned by the caller; the library never frees, retains or
 * reallocates caller memory.  All calls are asynchronous on `stream` (NULL
 * means the null stream) and return after enqueueing.  No call throws or
 * aborts: every failure is a negative status code.  Argument validation
 * happens on the host before any HIP call is made.
 */
#ifndef LIBMXGEMM_H
#define LIBMXGEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */

typedef int mxgemm_status;

#define MXGEMM_OK                      0
#define MXGEMM_ERR_INVALID_ARG        -1  /* NULL pointer, bad split_k, C == NULL with beta != 0, ... */
#define MXGEMM_ERR_SHAPE              -2  /* M, N < 1; K < 32; K % 32 != 0; K > 2^24; stride < extent */
#define MXGEMM_ERR_ALIGN              -3  /* A/B base not 16-byte aligned, or row pitch lda/2, ldb/2 not a multiple of 16 bytes */
#define MXGEMM_ERR_UNSUPPORTED_DEVICE -4  /* current device is not gfx950 */
#define MXGEMM_ERR_HIP                -5  /* a HIP runtime call failed (launch, allocation) */
#define MXGEMM_ERR_WORKSPACE          -6  /* caller workspace smaller than mxgemm_query's workspace_bytes */
#define MXGEMM_ERR_SCRATCH            -7  /* mxgemm_run_noalloc: the plan needs more than its fixed scratch */

/* Static string naming a status code (never NULL). */
const char *mxgemm_status_string(mxgemm_status status);

/* ---- strides and options --------------------------------------------------- */

/*
 * Row strides of the operands.  Passing NULL for the whole struct means
 * dense rows: ldd = ldc = N, lda = ldb = K, ldsa = ldsb = K/32, b_packed = 0,
 * library-owned workspace.
 *
 * The fully packed form (b_packed = sa_packed = 1: pre-shuffled B, shuffled
 * scaleA and scaleB, row-major A) is the operand set of the asm_f4gemm
 * README's pre-shuffled kernels ("Data layouts") and the fastest one: the
 * kernels read every shuffled scale word with contiguous loads.
 *
 * Units follow the asm_f4gemm README ("Kernel ABI", kernarg notes): A and B
 * strides count fp4 ELEMENTS (twice the byte pitch) and must be even; scale
 * strides count bytes; C and D strides count elements of their type.  ldc
 * and ldd are honoured separately, so D may alias C (in place) when ldc ==
 * ldd and C is bf16.
 *
 * The option fields at the end default to 0 (a zeroed struct):
 *   a_format   A's element format, MXGEMM_FMT_*: FP4 E2M1 (the default),
 *              FP8 E4M3, BF8 E5M2, FP6 E2M3 or FP6 E3M2 -- the inputs of the
 *              scaled matrix instructions ("CDNA4 dense MFMA builtins",
 *              "Mixed-precision with scaling"; encodings per the OCP MX
 *              v1.0 specification).  B stays FP4.  A row is a little-endian
 *              bit stream of the format's w-bit codes (element k at bits
 *              k*w .. k*w+w-1; for FP4 the low-nibble-first bytes), one E8M0
 *              scale per 32 elements as for FP4.  lda counts elements of
 *              A's format; the byte pitch lda*w/8 must be a whole multiple of
 *              16 (of 8 for the FP6 formats, whose dense rows are 24 bytes
 *              per 32 elements).  Kernels: for M == 1 the GEMV where it
 *              applies (kernel family 4), else for M <= 16 the
 *              skinny kernel, and for 16 < M <= 64 the rows kernel (all at
 *              the speed of
 *              the FP4 case; FP6 on the rows kernel needs an even K/32);
 *              otherwise, for M > 16, the 8-bit formats run on the tiled
 *              kernel with 8-bit A tiles, and FP6 A is first re-laid,
 *              codes unchanged, in a library-owned buffer per (device,
 *              stream), allocated on first use like the split-K buffers
 *              and freed by mxgemm_release_workspaces: on large shapes
 *              into the scaled instruction's operand order (24 bytes per
 *              lane, 1536 bytes per 16 rows and 128 K; its A scales
 *              shuffled beside it, and a row-major B and its scales packed
 *              as mxgemm_pack_b packs them) for a 256 x 256 FP6 tile,
 *              otherwise into 32-byte slots per 32-element block (rows of
 *              K bytes rounded up to 128) for the 8-bit tiles; both pass
 *              the FP6 operand format to the instruction, which runs it at
 *              its FP4 rate (when 256 re-laid rows reach 2^31 bytes, once
 *              per 16 rows on the skinny kernel instead).  Needs
 *              sa_packed = 0 and split_mode = MXGEMM_SPLIT_FP32 (else
 *              MXGEMM_ERR_INVALID_ARG); size a caller workspace with
 *              mxgemm_query_ex.
 *   c_f32      C is float32 instead of bf16.  The README's "C / bias" note
 *              says aiter documents its bias operand as f32; with c_f32 = 1
 *              the epilogue reads that type (D stays bf16; one rounding of
 *              alpha*acc + beta*C, computed in fp32).
 *   split_mode MXGEMM_SPLIT_FP32: split-K partials are fp32 sums added in a
 *              fixed order (deterministic; the default).
 *              MXGEMM_SPLIT_BF16_ATOMIC: each K chunk adds bf16(alpha *
 *              partial) into D with packed bf16 atomic adds, onto D first
 *              set to bf16(beta * C), the reduction the README's kernels use
 *              ("Verification": split-K accumulates in bf16).  Offered only
 *              to measure that reduction's error against the fp32 one: the
 *              result is rounded once per chunk and its bits depend on the
 *              order the chunks arrive in.  It runs on the tiled kernel
 *              (the skinny kernels are never chosen), needs D 4-byte
 *              aligned, ldd and N even (else MXGEMM_ERR_ALIGN), and D must
 *              not alias C.  With split 1 it is the ordinary path.
 *   b_layout   MXGEMM_B_NK: B as above ([N][ldb/2] rows, or mxgemm_pack_b's
 *              layout with b_packed = 1).  MXGEMM_B_KN: B's codes are
 *              stored MN-major, [K][ldb/2] bytes: row k holds the codes of
 *              the N columns at that k, element n in the low nibble of byte
 *              n/2 when n is even (a weight kept as W[K][N]).  ldb then
 *              counts fp4 elements between K-rows: ldb >= N, even, ldb/2 a
 *              multiple of 16 bytes.  scaleB stays one byte per column and
 *              32-block of k: [N][ldsb] with b_packed = 0, or
 *              mxgemm_pack_scales' shuffle of it over the N rows with
 *              b_packed = 1 (the codes are never pre-shuffled in this
 *              layout).  The tiled kernel reads such a B from LDS with the
 *              4-bit transposed loads of "CDNA4 MFMA transpose load
 *              builtins" (ds_read_tr4_b64, two per 16 x 128 operand, K
 *              split as that page's "Hardware constraints" table gives),
 *              for every M.  Needs a_format = MXGEMM_FMT_FP4 (else
 *              MXGEMM_ERR_INVALID_ARG); mxgemm_run_bf16a then quantizes
 *              first also at M = 1.
 */
#define MXGEMM_SPLIT_FP32        0
#define MXGEMM_SPLIT_BF16_ATOMIC 1

#define MXGEMM_B_NK 0  /* B [N][ldb/2]: row n holds its K codes (K-major) */
#define MXGEMM_B_KN 1  /* B [K][ldb/2]: row k holds the N columns' codes (MN-major) */

#define MXGEMM_FMT_FP4      0  /* E2M1, 4 bits */
#define MXGEMM_FMT_FP8_E4M3 1  /* 8 bits */
#define MXGEMM_FMT_FP8_E5M2 2  /* 8 bits */
#define MXGEMM_FMT_FP6_E2M3 3  /* 6 bits */
#define MXGEMM_FMT_FP6_E3M2 4  /* 6 bits */

typedef struct mxgemm_strides {
    int64_t ldd;      /* bf16 elements between rows of D, >= N */
    int64_t ldc;      /* elements between rows of C, >= N (ignored if beta == 0) */
    int64_t lda;      /* elements between rows of A (fp4 unless a_format says otherwise), >= K */
    int64_t ldb;      /* fp4 elements between rows of B, >= K (>= N for MXGEMM_B_KN), even
                         (ignored if b_packed with MXGEMM_B_NK) */
    int64_t ldsa;     /* bytes between rows of scaleA, >= K/32 */
    int64_t ldsb;     /* bytes between rows of scaleB, >= K/32 (ignored if b_packed) */
    int32_t b_packed; /* 0: B, scaleB row-major as above; 1: outputs of mxgemm_pack_b */
    int32_t sa_packed; /* 0: scaleA row-major as above; 1: output of mxgemm_pack_scales
                          for the M rows of A (ldsa ignored; needs b_packed = 1) */
    void *workspace;  /* optional device buffer for split-K partials; NULL = library-owned */
    size_t workspace_bytes;
    int32_t c_f32;      /* 0: C is bf16; 1: C is float32 */
    int32_t split_mode; /* MXGEMM_SPLIT_FP32 or MXGEMM_SPLIT_BF16_ATOMIC */
    int32_t a_format;   /* MXGEMM_FMT_* */
    int32_t b_layout;   /* MXGEMM_B_NK (B's rows hold K) or MXGEMM_B_KN (B's rows hold N) */
    int32_t a_packed;   /* 0: A and scaleA as above; 1: an FP6 A (a_format MXGEMM_FMT_FP6_*)
                           and its scales as mxgemm_pack_a wrote them (lda, ldsa and
                           sa_packed ignored; M > 64, where the dense FP6 tile runs; not
                           with mxgemm_run_bf16a): the call skips its re-layout of A */
} mxgemm_strides;

/* ---- the GEMM ------------------------------------------------------------- */

/*
 * D = bf16(alpha * A * B^T + beta * C).  Enqueued on `stream`.
 *
 * split_k: 0 or -1 lets the library choose (the "-1 lets the heuristic try"
 *          convention of the asm_f4gemm CLI, section "Build and run");
 *          1 = no split; 2, 4, 8 or 16 = split the K range into that many
 *          chunks whose fp32 partial sums are added in a fixed order (the
 *          result is bitwise reproducible run to run).  Other values:
 *          MXGEMM_ERR_INVALID_ARG.  Chunks are whole units of 256 K (tiled
 *          kernel, M > 64) or 512 K (skinny kernels, M <= 64); a split that
 *          needs smaller chunks is reduced to the number of such units
 *          (mxgemm_query reports the split used).
 *
 * Shapes: M, N >= 1; K >= 32, K % 32 == 0, K <= 2^24.  M and N need not be
 * multiples of any tile size and K need not be a multiple of 128: edges are
 * handled inside the kernels (no caller padding as in the asm_f4gemm README's
 * "D -- output" note).
 *
 * Alignment: A and B base addresses 16-byte aligned and lda/2, ldb/2 (the
 * byte pitches) multiples of 16.  Scales, C and D need only natural
 * alignment (D and a bf16 C: 2 bytes; an f32 C: 4 bytes).
 *
 * Split-K (split_k > 1, chosen or forced) keeps fp32 partial sums in a
 * workspace of mxgemm_query(...).workspace_bytes.  With strides->workspace
 * == NULL the library allocates one per (device, stream) on first use and
 * keeps it until mxgemm_release_workspaces(); a caller workspace must be at
 * least that size and must not be used by two calls that can run
 * concurrently.  The per-tile arrival counters of split-K are always
 * library-owned: one zeroed buffer per (device, stream), allocated on first
 * use and returned to all-zero by every call.  The first call with a new
 * (device, stream) or a larger need therefore allocates; calls on one
 * stream are ordered, calls on different streams use separate buffers.
 */
mxgemm_status mxgemm_run(void *D, const void *C, const void *A, const void *B,
                         const void *scaleA, const void *scaleB,
                         float alpha, float beta, int M, int N, int K,
                         const mxgemm_strides *strides, int split_k,
                         hipStream_t stream);

/* ---- allocation-free GEMM ------------------------------------------------------ */

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * mxgemm_run with every library-owned buffer taken from one fixed device
 * array per GPU of MXGEMM_NOALLOC_SCRATCH_BYTES (32 MiB), which the library
 * holds from load until the process ends: the split-K arrival counters
 * (first 64 KiB: 4 bytes per output tile of a split plan), the split-K fp32
 * partials unless strides->workspace brings them, and the re-laid copy of
 * an FP6 A on the tiled kernels (M * K bytes, K rounded up to 128, on the
 * 8-bit tiles; about 3/4 of that plus M * K / 32 scale bytes on the FP6
 * tile, plus N * K * 17/32 bytes when B is row-major).  Same
 * arguments, plans, kernels and results as
 * mxgemm_run, bit for bit.  Never calls hipMalloc or hipFree (the first call
 * on a device looks up that device's array once).  A plan that needs more
 * than the array holds returns MXGEMM_ERR_SCRATCH before any launch;
 * mxgemm_query_ex gives the plan's workspace_bytes.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents; each call clears the counters it uses (with a kernel on
 * `stream`) before its GEMM.  Calls that can overlap on one GPU (on
 * different streams, or from host threads without ordering) race on the
 * array and must not be issued; calls ordered on one stream are safe.
 */
#define MXGEMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

mxgemm_status mxgemm_run_noalloc(void *D, const void *C, const void *A, const void *B,
                                 const void *scaleA, const void *scaleB,
                                 float alpha, float beta, int M, int N, int K,
                                 const mxgemm_strides *strides, int split_k,
                                 hipStream_t stream);

/* ---- B pre-shuffle ----------------------------------------------------------- */

/*
 * Rewrite B [N][ldb/2] and scaleB [N][ldsb] into the layout the kernels read
 * directly (b_packed = 1).  The byte permutation is the "16x16
 * tile-transposed" B shuffle of the asm_f4gemm README ("Data layouts", B):
 *
 *   B[n0*16 + n1][k-byte k0*32 + k1*16 + k2]
 *       -> Bp[(((n0 * Kp/32 + k0) * 2 + k1) * 16 + n1) * 16 + k2],
 *
 * with Kp = (K rounded up to 128)/2 bytes and N rounded up to 16 rows, so
 * that every 1 KiB of Bp is one matrix-instruction operand (16 rows x 128
 * K), and the scale shuffle of the same section (its "A_scale / B_scale"
 * part), over scaleB padded to [N rounded up to 32][K/32 rounded up to 8]:
 *
 *   scaleB[d0*32 + d1*16 + d2][d3*8 + d4*4 + d5]
 *       -> SBp[((((d0 * sn/8 + d3) * 4 + d5) * 16 + d2) * 2 + d4) * 2 + d1],
 *
 * sn = padded K/32.  Padding bytes are code 0 for Bp and 0x7F (2^0) for SBp.
 * Bp and SBp are caller buffers of mxgemm_query's packed_b_bytes and
 * packed_sb_bytes; they must not overlap B or scaleB.  Bp 16-byte aligned,
 * SBp 4-byte aligned, B as for mxgemm_run.  Same shape rules as mxgemm_run.
 */
mxgemm_status mxgemm_pack_b(void *Bp, void *SBp, const void *B, const void *scaleB,
                            int N, int K, int64_t ldb, int64_t ldsb,
                            hipStream_t stream);

/*
 * Shuffle a [rows][K/32] E8M0 scale matrix (row pitch lds bytes) into the
 * layout of the asm_f4gemm README's "A_scale / B_scale" part of "Data
 * layouts" -- the same transform mxgemm_pack_b applies to scaleB -- for use
 * as scaleA with sa_packed = 1 (rows = M).  Sp is a caller buffer of
 * ceil(rows/32)*32 * ceil(K/256)*8 bytes (mxgemm_info.packed_sa_bytes for
 * rows = M), 4-byte aligned, not overlapping S; padding bytes are 0x7F.
 * Shape rules as mxgemm_run with rows in place of M.
 */
mxgemm_status mxgemm_pack_scales(void *Sp, const void *S, int rows, int K, int64_t lds,
                                 hipStream_t stream);

/*
 * An FP6 A (a_format MXGEMM_FMT_FP6_E2M3 or _E3M2; the layout does not depend
 * on which) and its scales, put once into the order the dense FP6 tile reads:
 * what mxgemm_run does to a row-major FP6 A on every call with M > 64
 * (for an A used in several calls, or written that way by its producer).
 * Codes: per 16-row group of A and 128-K step, 1536 bytes in the scaled
 * matrix instruction's operand order ("CDNA4 dense MFMA builtins",
 * "Mixed-precision with scaling": lane l holds row l%16, K-block l/16 of the
 * step, 24 bytes of FP6 codes, unchanged), steps padded to an even count,
 * groups in order; rows past M and blocks past K/32 are code 0.  Scales:
 * mxgemm_pack_scales' shuffle of scaleA (padding 0x7F).  A: [M][lda] FP6
 * elements (byte pitch lda*6/8 a multiple of 8; A 16-byte aligned);
 * scaleA: [M][ldsa] bytes.  Ap: mxgemm_pack_a_bytes(M, K) bytes, 16-byte
 * aligned; SAp: ceil(M/32)*32 * ceil(K/256)*8 bytes (packed_sa_bytes),
 * 4-byte aligned; neither overlaps A or scaleA.  Pass Ap as A and SAp as
 * scaleA to mxgemm_run with a_packed = 1.  Asynchronous on `stream`; errors
 * as mxgemm_run (MXGEMM_ERR_INVALID_ARG for another a_format).
 */
mxgemm_status mxgemm_pack_a(void *Ap, void *SAp, const void *A, const void *scaleA, int M, int K,
                            int64_t lda, int64_t ldsa, int a_format, hipStream_t stream);

/* Bytes of mxgemm_pack_a's Ap for an M x K FP6 A (0 for an invalid shape). */
size_t mxgemm_pack_a_bytes(int M, int K);

/* ---- activation quantizer -------------------------------------------------------- */

/*
 * Quantize a bf16 matrix X [M][ldx] (row-major, ldx in bf16 elements) to the
 * operand format of A: packed E2M1 codes A [M][lda/2] bytes (lda in fp4
 * elements, element 2i in the low nibble of byte i) and E8M0 scales
 * scaleA [M][ldsa] bytes, one per 32 consecutive K elements (asm_f4gemm
 * README, "Data layouts").  The outputs can be passed to mxgemm_run as A and
 * scaleA.
 *
 * The pages fix the encodings but not how a scale is chosen for real input;
 * the conversion follows the OCP Microscaling Formats v1.0 specification,
 * section 6.3: per 32-block, scale = 2^X with X = floor(log2 max|x|) - 2
 * clamped to [-127, 127]; each element is x / 2^X rounded to the nearest
 * E2M1 value (ties to the even mantissa), magnitudes beyond 6 saturate to 6,
 * the sign is kept (a negative value rounding to zero gives code 0x8).  A
 * block holding a NaN or an infinity gets scale 0xFF and codes 0; an all-zero
 * block gets scale 0x00 and codes 0.  The result is exact (deterministic and
 * independent of launch shape): every decision is taken on exactly scaled
 * values.
 *
 * Shapes: M >= 1; K >= 32, K % 32 == 0, K <= 2^24; ldx >= K, lda >= K,
 * ldsa >= K/32 (else MXGEMM_ERR_SHAPE).  Alignment (else MXGEMM_ERR_ALIGN):
 * X 16-byte aligned with ldx % 8 == 0; A 16-byte aligned with lda even and
 * lda/2 a multiple of 16 (the rule mxgemm_run applies to A); scaleA any.
 * X must not overlap A or scaleA.  Only the first K elements of each X row
 * are read and only the first K/2 bytes of each A row and K/32 bytes of each
 * scaleA row are written.  Asynchronous on `stream`; allocates nothing.
 */
mxgemm_status mxgemm_quantize(void *A, void *scaleA, const void *X, int M, int K,
                              int64_t ldx, int64_t lda, int64_t ldsa, hipStream_t stream);

/*
 * D = bf16(alpha * Q(X) * B^T + beta * C), where X is a bf16 activation
 * matrix [M][ldx] (row-major, ldx in bf16 elements, 16-byte aligned rows:
 * ldx % 8 == 0, X 16-byte aligned, ldx >= K) and Q is mxgemm_quantize's
 * encoding -- the activation-side quantizer in front of the GEMM.  B,
 * scaleB, C, D, strides (ldd, ldc, ldb, ldsb, b_packed, c_f32, workspace)
 * and split_k as for mxgemm_run; strides->lda / ldsa are ignored, and
 * a_format, sa_packed and split_mode must be 0 (else
 * MXGEMM_ERR_INVALID_ARG).
 *   M == 1 (decode), K-major B: one launch.  The skinny kernel loads the
 *     bf16 row and quantizes each 32-block in registers with the quantizer's
 *     rule, so D is bit for bit what mxgemm_quantize followed by mxgemm_run
 *     gives where mxgemm_run plans the skinny kernel too; where it plans the
 *     single-row GEMV (kernel family 4, another K order) the two agree
 *     within the fp32 accumulation's rounding.
 *   M > 1, or an MN-major B (b_layout = MXGEMM_B_KN): mxgemm_quantize into a library-owned buffer of
 *     M*K/2 + M*K/32 bytes per (device, stream) (allocated on first use like
 *     the split-K buffers, freed by mxgemm_release_workspaces), then
 *     mxgemm_run on it, both on `stream`.
 * Asynchronous on `stream`; errors as mxgemm_run.
 */
mxgemm_status mxgemm_run_bf16a(void *D, const void *C, const void *X, const void *B, const void *scaleB,
                               float alpha, float beta, int M, int N, int K, int64_t ldx,
                               const mxgemm_strides *strides, int split_k, hipStream_t stream);

/* ---- FP16 GEMM with transposed LDS reads ---------------------------------- */

/*
 * C = A * B with A [M, K] fp16 row-major, B [K, N] fp16 row-major (K-major:
 * row k holds the N columns of that k) and C [M, N] fp32: the FP16 GEMM of
 * "CDNA4 MFMA transpose load builtins" ("FP16 GEMM example"), whose B
 * fragments are read from LDS with ds_read_tr16_b64 (a hardware 16-bit
 * transpose) because B is stored K-major.  Products are exact in fp32 and
 * accumulate in fp32 inside the v_mfma_f32_16x16x32_f16 instructions.
 *
 * Strides count elements: lda >= K, ldb >= N, ldc >= N.  Shapes: M, N, K
 * >= 1, K and N multiples of 8 (whole 16-byte chunks of the rows of A and
 * B), 256 * lda * 2 and K * ldb * 2 below 2^31 bytes.  A, B base 16-byte
 * aligned, lda and ldb multiples of 8; C 4-byte aligned.  Errors:
 * MXGEMM_ERR_INVALID_ARG (NULL pointer), MXGEMM_ERR_SHAPE, MXGEMM_ERR_ALIGN,
 * all before any HIP call.  Asynchronous on `stream`; allocates nothing.
 */
mxgemm_status mxgemm_f16_run(void *C, const void *A, const void *B, int M, int N, int K,
                             int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream);

/* ---- plan / query ------------------------------------------------------------- */

typedef struct mxgemm_info {
    int32_t kernel;          /* kernel family: 0 = tiled (LDS, M > 64); 1 = skinny (M <= 16,
                                streams B); 2 = skinny rows (16 < M <= 64, streams B, A
                                shared through LDS); 3 = tiled with an FP8/FP6 A; 4 =
                                GEMV (M == 1, or 2 <= M <= 8 with FP4 A; row-major B,
                                K % 2048 == 0, N >= 4 x num_cu, unsplit; 4 rows of B per
                                workgroup; with 16-byte aligned scale rows, else the skinny
                                kernel) */
    int32_t tile_m, tile_n;  /* output tile per workgroup */
    int32_t split_k;         /* K chunks the plan uses */
    int64_t grid;            /* workgroups launched */
    size_t workspace_bytes;  /* split-K fp32 partials workspace needed (0 if split_k == 1) */
    size_t packed_b_bytes;   /* size of mxgemm_pack_b's Bp for this N, K */
    size_t packed_sb_bytes;  /* size of mxgemm_pack_b's SBp for this N, K */
    size_t packed_sa_bytes;  /* size of mxgemm_pack_scales' output for the M rows of scaleA */
    int32_t num_cu;          /* compute units the plan assumed */
    int32_t persist_grid;    /* > 0: the tiled kernel runs persistent, this many workgroups
                                (one per CU) walking the `grid` tiles in the same order;
                                assumes beta == 0 and 16-byte aligned pointers, as the
                                persistent form needs (else mxgemm_run uses the plain grid) */
    char kernel_name[64];
    char arch[32];           /* device architecture (mxgemm_query only) */
    double peak_flops;       /* dense MXFP4 matrix peak, flop/s, from the device clock and CU count */
    double clock_hz;         /* peak engine clock used for peak_flops */
} mxgemm_info;

/*
 * Plan for the current device: the kernel, tile and split mxgemm_run would
 * use for these arguments, and the buffer sizes it needs.  The plan follows
 * the asm_f4gemm README's "Tile selection heuristic" (count the rounds of
 * workgroups the compute units need per tile shape, prefer fewer rounds of
 * larger tiles, iterate candidates in a fixed order), weighted by a per-tile
 * cost that also prices split-K.  Returns MXGEMM_ERR_UNSUPPORTED_DEVICE
 * unless the current device is gfx950.  split_k as for mxgemm_run.
 */
mxgemm_status mxgemm_query(int M, int N, int K, int b_packed, int split_k,
                           mxgemm_info *out);

/*
 * The same plan for a device with num_cu compute units, computed on the
 * host without touching any device (arch, peak_flops, clock_hz left 0).
 */
mxgemm_status mxgemm_plan(int M, int N, int K, int b_packed, int split_k, int num_cu,
                          mxgemm_info *out);

/* mxgemm_plan / mxgemm_query for the exact path mxgemm_run takes with these
 * strides and options (a_format, split_mode, b_packed; NULL = defaults):
 * with a wider A format or the bf16-atomic split the kernel and the
 * workspace differ from the FP4 plan, and a caller workspace must be sized
 * from this call.  kernel = 3 is the tiled kernel with 8-bit A.  Same
 * errors as mxgemm_plan / mxgemm_query, plus MXGEMM_ERR_INVALID_ARG for
 * option values mxgemm_run rejects. */
mxgemm_status mxgemm_plan_ex(int M, int N, int K, const mxgemm_strides *strides, int split_k, int num_cu,
                             mxgemm_info *out);
mxgemm_status mxgemm_query_ex(int M, int N, int K, const mxgemm_strides *strides, int split_k,
                              mxgemm_info *out);

/* ---- measurement ------------------------------------------------------------ */

/*
 * Read `bytes` of device memory at src once, with the 16-byte non-temporal
 * loads the skinny kernels stream B with, and nothing else (sink, a 4-byte
 * device word, is written only if the XOR of everything read equals a fixed
 * constant).  A kernel whose minimum DRAM traffic is `bytes` cannot finish
 * faster on this chip ("Optimizing GEMM in HIP", background: the GEMM's
 * arithmetic intensity against its minimum required traffic), so its time
 * is the achievable ceiling the benchmark reports next to the published HBM
 * bandwidth.  bytes: a multiple of 16, below 2^31 (else
 * MXGEMM_ERR_SHAPE); src 16-byte and sink 4-byte aligned (else
 * MXGEMM_ERR_ALIGN).  Asynchronous on `stream`; allocates nothing.
 */
mxgemm_status mxgemm_stream_read(const void *src, size_t bytes, void *sink, hipStream_t stream);

/* Free the library-owned split-K workspaces (after synchronizing their
 * streams).  Later calls allocate again. */
mxgemm_status mxgemm_release_workspaces(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMXGEMM_H */
