/*
 * jq4k.h -- Q4_K weight-only matmul for AMD Instinct MI355X (gfx950).
 *
 * The operation.  The genie-ai-runtime README ("At a glance"; "Project
 * layout", src/kernels/) names the two hot kernels of its GGUF engine: an
 * "INT4 dequant-fused GEMV" for decode and a "tensor-core MMQ Q4_K prefill"
 * matmul, run on the Qwen3-4B-Q4_K_M model.  Both compute, for every linear
 * projection of the model,
 *
 *        Y[m][n] = sum_k  w[n][k] * x[m][k]        (Y = X . W^T)
 *
 * where W is stored in GGUF's Q4_K format and dequantised on the fly.
 *
 * Q4_K block (GGUF): 256 weights in 144 bytes,
 *     d, dmin        binary16 super-block scale and min (little-endian)
 *     scales[12]     eight 6-bit sub-block scales sc_j and eight 6-bit mins
 *                    m_j: j < 4 in the low six bits of scales[j] / scales[j+4];
 *                    j >= 4 low nibbles in scales[j+4] (sc low, m high) and
 *                    top two bits in bits 6..7 of scales[j-4] (sc) / scales[j] (m)
 *     qs[128]        4-bit quants: weight i in byte 32*(i/64) + i%32, low
 *                    nibble when (i/32) is even, high nibble otherwise
 *     w_i = d * sc_s * q_i - dmin * m_s,   s = i / 32.
 *
 * Layouts (all dense, row-major, no leading-dimension arguments):
 *     W  N rows x K/256 blocks; row n is output feature n:  W[n*(K/256) + kb]
 *     X  M x K bfloat16 (raw bit patterns)
 *     Y  M x N fp32
 *
 * Numerics.  Y is overwritten (never accumulated into).  Results are
 * deterministic: the same inputs on the same device give bit-identical Y.
 * The accuracy contract is |y - y_ref| <= 2e-3 * sum_k |w*x| + 1e-5 per
 * element, y_ref the exact contraction of the fp32 dequantised weights (see
 * jq4k_dequant_f32).
 *   M = 1 (jq4k_gemv, jq4k_gemv_batched, jq4k_gemv_rmsnorm, jq4k_gemm_swiglu
 *   at M = 1): every output meets the contract.  The kernel sums each
 *   sub-block in factored form, d*sc * sum(q x) - dmin*m * sum(x), with
 *   exact products (x staged as binary16 times a power of two per block of
 *   256) and fp32 sums, and bounds each row's rounding error from the same
 *   data: at most (192 + K/256) * 2^-24 * sum over sub-blocks of
 *   (15 |d sc| + |dmin m|) * sum |x|.  A row whose bound does not certify
 *   2e-3 * sum|w*x| + 1e-5 against a lower bound of sum|w*x| (weights near
 *   zero against large scales, e.g. d*sc*q = dmin*m) is recomputed in the
 *   same launch from the fp32 weights with fp64 sums, as are all rows when
 *   an activation is not exact in its staged binary16 (a value below 2^-31
 *   of its block's largest magnitude, Inf, NaN).  The bound assumes each
 *   dot-product step adds its two exact binary16 products to the fp32 sum
 *   with at most two roundings.  Rows of randomly drawn Q4_K blocks
 *   certify with a margin of about 8 and are never recomputed.
 *   M > 1: the matrix-core kernels contract bfloat16 tiles of w
 *   (round-to-nearest-even of the fp32 weight, exactly what
 *   jq4k_dequant_bf16 returns) with fp32 accumulation.  bfloat16 keeps 8
 *   significant bits (relative error up to 2^-8), so adversarial blocks whose
 *   weights all sit near a bfloat16 rounding midpoint, against activations of
 *   one sign, can exceed the 2e-3 term by up to about 2x; randomly drawn
 *   Q4_K weights stay far inside it.
 * Inf/NaN in d, dmin or x propagate per IEEE.
 *
 * Ownership and execution.  All pointers are device pointers owned by the
 * caller; the library allocates no memory and keeps no state beyond a cache
 * of device attributes.  Work is enqueued on `stream` (0 = the null stream);
 * nothing synchronises with the host, so errors raised while the kernel runs
 * surface at the caller's next synchronisation.  Calls are thread-safe.
 *
 * Return codes.  0 on success.  JQ4K_EINVAL / JQ4K_EALIGN when the arguments
 * are rejected -- checked before any HIP call, so nothing is launched.  A
 * positive value is the hipError_t reported when the launch failed.
 */
#ifndef JQ4K_H
#define JQ4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as in HIP's runtime headers. */
typedef struct ihipStream_t *hipStream_t;

typedef struct {
    uint16_t d;          /* binary16 bits */
    uint16_t dmin;       /* binary16 bits */
    uint8_t scales[12];
    uint8_t qs[128];
} block_q4_K;

#ifdef __cplusplus
static_assert(sizeof(block_q4_K) == 144, "block_q4_K must be 144 bytes");
#else
_Static_assert(sizeof(block_q4_K) == 144, "block_q4_K must be 144 bytes");
#endif

typedef uint16_t jq4k_bf16; /* bfloat16 bit pattern */
typedef uint16_t jq4k_f16;  /* IEEE binary16 bit pattern */

#define JQ4K_OK 0
#define JQ4K_EINVAL (-1) /* bad size, null pointer with a nonzero size,  */
                         /* K not a positive multiple of 256, M != 1 for */
                         /* the GEMV, K above the GEMV limit, bad path   */
#define JQ4K_EALIGN (-2) /* W or X not 16-byte aligned, Y not 4-byte    */
#define JQ4K_ESCRATCH (-3) /* jq4k_gemm_batched_noalloc: the problems   */
                           /* need more than JQ4K_SCRATCH_BYTES          */

/* Largest K the M = 1 kernel accepts (it keeps x in LDS). */
#define JQ4K_GEMV_MAX_K 16384

/* Largest K the matrix-core kernels accept (a tile of X rows is addressed
 * with 32-bit byte offsets). */
#define JQ4K_MFMA_MAX_K 4194304

/* Decode GEMV, M must be 1: Y[0..N) = sum_k w[n][k] * X[k].
 * The genie-ai-runtime README, "At a glance": INT4 dequant-fused GEMV.
 * W: N*(K/256) blocks, 16-byte aligned.  X: K bf16, 16-byte aligned.
 * Y: N floats, 4-byte aligned.  N == 0 returns 0 without launching.
 * Errors: JQ4K_EINVAL for M != 1, N < 0, K <= 0, K % 256 != 0,
 * K > JQ4K_GEMV_MAX_K, or a null pointer; JQ4K_EALIGN for misalignment. */
int jq4k_gemv(const block_q4_K *W, const jq4k_bf16 *X, float *Y,
              int M, int N, int K, hipStream_t stream);

/* jq4k_gemv for one token with an explicit number of rows of W per
 * workgroup (a tuning knob; 0 picks the same value jq4k_gemv uses).  Larger
 * values stage x fewer times, smaller ones spread a small matrix over more
 * compute units.  JQ4K_EINVAL for rows_per_block < 0 or a value whose LDS
 * need exceeds 96 KiB; otherwise the same rules as jq4k_gemv with M = 1. */
int jq4k_gemv_rows(const block_q4_K *W, const jq4k_bf16 *X, float *Y,
                   int N, int K, int rows_per_block, hipStream_t stream);

/* One problem of a batched decode GEMV: Y[0..N) = sum_k w[n][k] * X[k]. */
typedef struct {
    const block_q4_K *W;  /* N*(K/256) blocks, 16-byte aligned */
    const jq4k_bf16 *X;   /* K bf16, 16-byte aligned           */
    float *Y;             /* N floats, 4-byte aligned          */
    int N;
    int K;                /* positive multiple of 256, <= JQ4K_GEMV_MAX_K */
} jq4k_gemv_desc;

#define JQ4K_GEMV_BATCH_MAX 16

/* Up to JQ4K_GEMV_BATCH_MAX independent decode GEMVs in one kernel launch
 * (the genie-ai-runtime README, "At a glance": INT4 dequant-fused GEMV; one
 * launch for the projections of a layer that do not depend on each other,
 * such as q, k and v, or gate and up).  Each problem gets exactly the result
 * jq4k_gemv gives for it; problems with N == 0 are skipped.  `problems` is a
 * host array read before the call returns (the descriptors are passed to the
 * kernel by value; nothing is allocated).  Outputs must not overlap any
 * input.  Errors: JQ4K_EINVAL for count < 0, count > JQ4K_GEMV_BATCH_MAX, a
 * null `problems` with count > 0, or any problem that jq4k_gemv rejects
 * (JQ4K_EALIGN likewise); nothing is launched then. */
int jq4k_gemv_batched(const jq4k_gemv_desc *problems, int count, hipStream_t stream);

/* Matmul for any M >= 0: Y (M x N) = X (M x K) . W^T.
 * The genie-ai-runtime README, "At a glance": tensor-core MMQ Q4_K prefill.
 * M == 1 runs the decode GEMV when K <= JQ4K_GEMV_MAX_K; 2 <= M <= 64 the
 * small-M MFMA kernel (W dequantised in registers, whole K per workgroup);
 * larger M the dequantise-to-LDS bf16 MFMA kernels (K <= JQ4K_MFMA_MAX_K,
 * else JQ4K_EINVAL): 128-row tiles, or the wave-specialised 256-row tile from
 * M = 2048, and from M = 512 when the matmul still gives every compute unit
 * two 256 x 128 tiles; a 256-row launch whose 256 x 256 output tiles give
 * every compute unit at least three runs the register-W kernel
 * (JQ4K_PATH_MFMA_RW) instead.  M == 0 or N == 0 returns 0 without
 * launching.  Same pointer and alignment rules as jq4k_gemv. */
int jq4k_gemm(const block_q4_K *W, const jq4k_bf16 *X, float *Y,
              int M, int N, int K, hipStream_t stream);

/* One problem of a batched matmul: Y (M x N) = X (M x K) . W^T. */
typedef struct {
    const block_q4_K *W;  /* N*(K/256) blocks, 16-byte aligned */
    const jq4k_bf16 *X;   /* M x K bf16, 16-byte aligned       */
    float *Y;             /* M x N floats, 4-byte aligned      */
    int M;
    int N;
    int K;                /* positive multiple of 256          */
} jq4k_gemm_desc;

#define JQ4K_GEMM_BATCH_MAX 16

/* Up to JQ4K_GEMM_BATCH_MAX independent matmuls in one launch on the MFMA
 * path (the genie-ai-runtime README, "At a glance": tensor-core MMQ Q4_K
 * prefill; one launch for projections that do not depend on each other, such
 * as q, k and v, or gate and up, so that their tiles fill the GPU together).
 * The tile (64, 128 or 256 rows of M) follows the largest M of the batch:
 * 64 up to M = 64, 256 from M = 512, else 128; a 256-row batch whose
 * 256 x 256 output tiles give every compute unit at least three runs the
 * register-W kernel.  Every problem meets the same bounds as jq4k_gemm.
 * Problems
 * with M == 0 or N == 0 are skipped.  `problems` is a host array read before
 * the call returns (passed to the kernel by value; nothing is allocated).
 * Outputs must not overlap any input.  Errors: JQ4K_EINVAL for count < 0,
 * count > JQ4K_GEMM_BATCH_MAX, a null `problems` with count > 0, or any
 * problem that jq4k_gemm rejects (JQ4K_EALIGN likewise); nothing is launched
 * then. */
int jq4k_gemm_batched(const jq4k_gemm_desc *problems, int count, hipStream_t stream);

/* Grouped matmul with a caller-provided workspace, for the small-M (M <= 64)
 * launches (the genie-ai-runtime README, "At a glance": tensor-core MMQ Q4_K
 * prefill, here at the short-prompt sizes).  There each output tile is only
 * 64 wide and a long row of W (K = 9728, say) would keep one workgroup busy
 * after the others finish; instead the K of such problems is cut into ranges
 * of whole blocks, one workgroup each (and a small problem may be cut in two
 * so that the workgroups left after the last full round of resident ones
 * are half ranges, not whole tiles).  Each range writes an fp32 partial tile
 * to the workspace and the last to finish adds them in range order, so the
 * result is the same whichever finishes last, run to run.  Same problems,
 * results and errors as jq4k_gemm_batched; when no problem is split (M > 64,
 * or nothing to gain) this is jq4k_gemm_batched and the workspace is unused.
 *   workspace        device memory of at least the size that
 *                    jq4k_gemm_workspace_size reports for the same problems,
 *                    256-byte aligned, all zero before its first use; each
 *                    call leaves it ready for the next (its counters back at
 *                    zero once the call completes).  Owned by the caller.
 *   workspace_bytes  its size.
 * Calls that may run at the same time (other streams) need workspaces of
 * their own.  Errors, besides jq4k_gemm_batched's: JQ4K_EINVAL if a
 * workspace is needed and `workspace` is null or smaller than needed,
 * JQ4K_EALIGN if it is not 256-byte aligned; nothing is launched then. */
int jq4k_gemm_batched_ws(const jq4k_gemm_desc *problems, int count, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Size of the static device buffer jq4k_gemm_batched_noalloc uses as its
 * split-K workspace (one per GPU, held until the process ends). */
#define JQ4K_SCRATCH_BYTES (8u << 20)

/* jq4k_gemm_batched_ws without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The split K workspace is a static
 * device array of JQ4K_SCRATCH_BYTES per GPU; nothing is allocated (no
 * hipMalloc, no allocating library call).  The first call on a device looks
 * up that device's copy and clears it once on `stream`.  Same problems,
 * results and errors as jq4k_gemm_batched_ws (bit-identical outputs), plus
 * JQ4K_ESCRATCH, with nothing launched, when jq4k_gemm_workspace_size would
 * exceed JQ4K_SCRATCH_BYTES for these problems (a Qwen3-4B layer at M <= 64
 * needs 1.8 MB, its down projection alone 6.6 MB).  Every call on one GPU
 * shares that GPU's buffer: calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. */
int jq4k_gemm_batched_noalloc(const jq4k_gemm_desc *problems, int count, hipStream_t stream);

/* Workspace bytes jq4k_gemm_batched_ws needs for these problems (0 when no
 * problem splits K; the size depends on the shapes and on the number of
 * compute units of the current device).  Host only, launches nothing.
 * Errors: those of jq4k_gemm_batched for the problems (with *bytes = 0),
 * JQ4K_EINVAL for a null `bytes`. */
int jq4k_gemm_workspace_size(const jq4k_gemm_desc *problems, int count, size_t *bytes);

/* Decode GEMV with the RMSNorm of x fused into its staging (the
 * genie-ai-runtime README, "At a glance": fused RMSNorm + RoPE + SwiGLU;
 * Qwen3's RMSNorm ahead of a projection):
 *   x_hat[k] = bf16(x[k] / sqrt(mean_k(x^2) + eps) * gamma[k]),  Y = W . x_hat.
 * x_hat is rounded to bf16 (nearest even) as an activation stored between
 * the two steps would be; the sum of squares is reduced in fp32 in a fixed
 * order.  X and gamma: K bf16 each, 16-byte aligned.  Errors: JQ4K_EINVAL
 * for eps < 0, eps infinite or NaN, a null gamma, or what jq4k_gemv rejects
 * with M = 1; JQ4K_EALIGN for a misaligned gamma or as jq4k_gemv.  N == 0
 * returns 0 without launching. */
int jq4k_gemv_rmsnorm(const block_q4_K *W, const jq4k_bf16 *X, const jq4k_bf16 *gamma,
                      float eps, float *Y, int N, int K, hipStream_t stream);

/* RMSNorm of M bf16 activation rows ahead of a prefill projection (the
 * genie-ai-runtime README, "At a glance": fused RMSNorm + RoPE + SwiGLU
 * kernels; the norm is Qwen3's): Xhat[m][k] = bf16(X[m][k] * r_m * gamma[k]),
 * r_m = 1 / sqrt(mean_k X[m][k]^2 + eps), computed in fp32 with the same
 * reduction order and products as jq4k_gemv_rmsnorm, so that composing it
 * with jq4k_gemv gives that function's result.  X and Xhat are M x K
 * row-major, gamma K values; Xhat may be X itself (in place), any other
 * overlap is undefined.  Feed Xhat to jq4k_gemm / jq4k_gemm_batched: at
 * M > 1 the rows are normalised once here rather than in every matmul
 * workgroup.  Errors: JQ4K_EINVAL for M < 0, K not a positive multiple of
 * 256 or K > JQ4K_GEMV_MAX_K, eps < 0, infinite or NaN, or a null pointer
 * with M > 0; JQ4K_EALIGN unless X, gamma and Xhat are 16-byte aligned.
 * M == 0 returns 0 without launching. */
int jq4k_rmsnorm_bf16(const jq4k_bf16 *X, const jq4k_bf16 *gamma, float eps, jq4k_bf16 *Xhat,
                      int M, int K, hipStream_t stream);

/* SwiGLU of a gate/up projection pair, one launch for any M >= 0:
 * H (M x N) = silu(X . Wg^T) * (X . Wu^T), elementwise, silu(z) = z / (1 +
 * exp(-z)) (the genie-ai-runtime README, "At a glance": fused RMSNorm + RoPE
 * + SwiGLU; the activation of Qwen3's MLP).  Wg and Wu are N rows of K/256
 * blocks each; the gate and up products are never written.  M == 1 with
 * K <= JQ4K_GEMV_MAX_K runs the decode GEMV over both matrices; larger M the
 * MFMA kernels (K <= JQ4K_MFMA_MAX_K), each tile holding the gate and up
 * columns of the same outputs.  Accuracy: each of g and u within the
 * matmul's bound, then silu and the product in fp32.  M == 0 or N == 0
 * returns 0 without launching.  Errors: JQ4K_EINVAL / JQ4K_EALIGN under the
 * rules of jq4k_gemm, applied to both matrices; H must not overlap an
 * input. */
int jq4k_gemm_swiglu(const block_q4_K *Wg, const block_q4_K *Wu, const jq4k_bf16 *X, float *H,
                     int M, int N, int K, hipStream_t stream);

/* Kernel paths for jq4k_gemm_path (tests and benchmarks reach every path). */
#define JQ4K_PATH_AUTO 0 /* what jq4k_gemm picks                        */
#define JQ4K_PATH_GEMV 1 /* the M = 1 kernel (M must be 1)               */
#define JQ4K_PATH_MFMA 2 /* the MFMA kernels, chosen by shape (M <= 64:  */
                         /* the small-M kernel)                         */
#define JQ4K_PATH_MFMA_T64 3  /* MFMA kernel, 64-row M tile              */
#define JQ4K_PATH_MFMA_T128 4 /* MFMA kernel, 128-row M tile             */
#define JQ4K_PATH_MFMA_T256 5 /* MFMA kernel, 256-row M tile, eight waves  */
                              /* (four dequantise, four multiply)         */
#define JQ4K_PATH_SKINNY 6    /* small-M MFMA kernel (M <= 64), whole K;  */
                              /* W dequantised in registers, X in LDS     */
#define JQ4K_PATH_MFMA_BIG 7  /* MFMA kernel, 256 x 256 tiles, four waves */
                              /* that each load, dequantise and multiply  */
#define JQ4K_PATH_MFMA_RW 8   /* MFMA kernel, 256 x 256 tiles, four waves */
                              /* that dequantise W into operand registers */

/* jq4k_gemm with an explicit kernel path; JQ4K_EINVAL for an unknown path,
 * JQ4K_PATH_GEMV with M != 1 or JQ4K_PATH_SKINNY with M > 64.  Results meet
 * the same bound on every path. */
int jq4k_gemm_path(const block_q4_K *W, const jq4k_bf16 *X, float *Y,
                   int M, int N, int K, int path, hipStream_t stream);

/* ---- FP16 <-> INT8 KV-cache convert (the genie-ai-runtime README,
 * "Project layout": FP16<->INT8 KV convert; "At a glance": INT8 KV cache by
 * default, FP16-ULP-bounded drift).  The pages give no scheme; the one here:
 * each KV vector (dim binary16 values, e.g. one token's head) has one fp32
 * scale s = max|v| / 127 and int8 codes q = rint(v / s) (round half to even,
 * q = 0 when s = 0); dequantised values are fp16(fp32(q * s)), round to
 * nearest even.  Each step is one IEEE operation, so codes, scales and
 * values are fixed bit for bit.  Contract (for vectors with max|v| >= 2^-14,
 * the binary16 normal range): |v' - v| <= s / 2 (plus half a binary16 ulp of
 * v'), and quantising v' again gives the same codes (no drift beyond the
 * first round trip).  Non-finite inputs are outside the contract. */
#define JQ4K_KV_MAX_DIM 512

/* Quantise nvec vectors of dim binary16 values.
 *   v      device, nvec * dim values, row-major, 16-byte aligned
 *   q      device, nvec * dim int8 codes (same layout), 8-byte aligned
 *   scale  device, nvec fp32 scales, 4-byte aligned
 *   dim    a multiple of 8, 8 <= dim <= JQ4K_KV_MAX_DIM
 * nvec == 0 returns 0 without launching.  Errors: JQ4K_EINVAL (nvec < 0, bad
 * dim, a null pointer, a size that overflows), JQ4K_EALIGN; nothing is
 * launched then. */
int jq4k_kv_quant_i8(const jq4k_f16 *v, int8_t *q, float *scale, long nvec, int dim,
                     hipStream_t stream);

/* Dequantise: v[r][i] = fp16(fp32(q[r][i] * scale[r])).  Same sizes, layouts,
 * alignment and errors as jq4k_kv_quant_i8. */
int jq4k_kv_dequant_f16(const int8_t *q, const float *scale, jq4k_f16 *v, long nvec, int dim,
                        hipStream_t stream);

/* Test exports.  They run the same device unpacking code as the matmul
 * kernels, one block per 256 outputs, so their outputs pin that code.
 *   jq4k_unpack_fields: q[256*nblocks] (0..15), sc[8*nblocks], m[8*nblocks]
 *                       (0..63), in block order; byte outputs need no
 *                       alignment.
 *   jq4k_dequant_f32:   w[256*nblocks], the fp32 weight d*sc*q - dmin*m
 *                       rounded once (round-to-nearest-even); 4-byte aligned.
 *   jq4k_dequant_bf16:  w[256*nblocks], bfloat16 of that fp32 weight
 *                       (round-to-nearest-even), the values the MFMA path
 *                       multiplies; 4-byte aligned.
 * W must be 16-byte aligned.  nblocks == 0 returns 0; nblocks < 0 or null
 * pointers give JQ4K_EINVAL. */
int jq4k_unpack_fields(const block_q4_K *W, long nblocks, uint8_t *q,
                       uint8_t *sc, uint8_t *m, hipStream_t stream);
int jq4k_dequant_f32(const block_q4_K *W, long nblocks, float *w,
                     hipStream_t stream);
int jq4k_dequant_bf16(const block_q4_K *W, long nblocks, jq4k_bf16 *w,
                      hipStream_t stream);

/* Text for a return code (static storage). */
const char *jq4k_strerror(int code);

/* Library version, major * 10000 + minor * 100 + patch. */
int jq4k_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JQ4K_H */
