/*
 * q4k.h -- C ABI of libq4k.so: fused Q4_K dequantize-and-multiply on MI355X
 * (gfx950), hand-written HIP kernels.
 *
 * The operation.  "Struct WgslForwardPass" (trueno docs), upload_q4k_weight:
 * weights stay as raw Q4K bytes and are multiplied by a fused dequant+GEMV on
 * the GPU.  "qualia_core_db/inference/cuda_lane/mod.rs" names the entry points
 * this ABI mirrors (try_q4k_soa_gemv, try_q4k_soa_fused_swiglu) and, under
 * "Honest limits", the fallback they replace: dequantize once to dense f32.
 *
 * Weight format.  A Q4_K matrix W of n rows and k columns (k % 256 == 0) is
 * n * (k/256) super-blocks of 144 bytes, row-major: row r occupies bytes
 * [r*(k/256)*144, (r+1)*(k/256)*144) and its super-block b covers columns
 * [256b, 256b+256) ("@simulatte/doppler 0.1.7 -> 0.1.8", matmul.d.ts,
 * MatmulOptions.transposeB: B is [N,K], row-major).  A super-block is
 *     bytes 0-1   d      IEEE binary16, little-endian
 *     bytes 2-3   dmin   IEEE binary16, little-endian
 *     bytes 4-15  eight six-bit scales sc_j and eight six-bit mins m_j
 *     bytes 16-143 256 four-bit codes q (byte 32g+l: low nibble is weight
 *                  64g+l, high nibble weight 64g+32+l)
 * and weight e of sub-block j = e/32 is  w = d*sc_j*q - dmin*m_j  (the GGUF
 * Q4_K layout; the pages' model files are Q4_K_M GGUF files, issue #3346).
 *
 * Conventions shared by every entry point:
 *  - All pointers except `stream` are DEVICE pointers owned by the caller.
 *    Every call only enqueues work on `stream` (a hipStream_t passed as
 *    void*; NULL means the null stream) and returns; it never synchronises.
 *    Results are ready when the stream is.  Only the batched calls on the
 *    matrix cores (see q4k_gemv_batched) and the prefill GEMM need device
 *    scratch, about 67 * ceil(m'/16) * k bytes for the batched call with
 *    m' = min(m, 64) tokens (about 1.1 MB at m = 64, k = 4096; the size
 *    queries below give it exactly).  Called plainly they use a buffer the
 *    library keeps per (device, stream), allocated stream-ordered from the
 *    device's default memory pool (hipMallocAsync on `stream`) the first time
 *    a stream needs it and grown the same way when a call needs more; calls
 *    on one stream run in order and calls on different streams use different
 *    buffers.  The buffers are held until the process ends (up to 64 MiB
 *    per stream, 64 streams); beyond that, and while `stream` is being
 *    captured into a graph, a call allocates and frees its own scratch
 *    stream-ordered.  Through their *_ws forms the scratch is a workspace
 *    the caller passes in, and q4k_gemv_batched_noalloc uses a static array.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched and the status says why.  Launch failures are
 *    reported as Q4K_ERR_LAUNCH.
 *  - w must be 16-byte aligned; x, y, h must be 4-byte aligned and the
 *    dequant output 16-byte aligned.  Outputs
 *    must not overlap any input.  Sub-ranges of rows are passed by pointer
 *    offsets (w + r0*(k/256)*144, y + r0), which keep 16-byte alignment.
 *  - n == 0 or m == 0 is an empty call: Q4K_OK, nothing launched.  k == 0 is
 *    a valid empty sum: outputs are written as 0 (dequant writes nothing).
 *  - Activations and outputs are f32, except where a call takes a q4k_dtype
 *    (and the prefill GEMM, whose activations are f16).  The products use the
 *    factored form sum_j [d*sc_j * sum_{e in j} q_e x_e - dmin*m_j * sum_{e in
 *    j} x_e], with the activations of each token in block fixed point.
 *  - Accuracy.  For one output write A = sum_k |w_k x_k| and B = sum_k
 *    (|d| sc_k q_k + |dmin| m_k) |x_k| (the two factored terms of each weight
 *    counted apart).  Each group of 64 consecutive activations of a token
 *    (128 on the matrix cores) is held to about 22 bits relative to its
 *    largest |x|.  Before any product the kernels compare each group's total
 *    rounding E with S4, the sum of the group's |x| other than its four
 *    largest; where E exceeds 2^-15 S4 (a few outliers far above the rest of
 *    their group, say) that group is multiplied in f32 instead, every weight
 *    dequantized on its own and every product rounded once.  Every result
 *    therefore satisfies
 *        |y - y_exact| <= 2^-15 sum_g max_{k in g} |w_k| S4_g + cB B + cA A
 *    with cB = 2^-22, cA = 2^-18 on the batch-1 and few-token kernels
 *    (groups of 64), and cB = 2^-18 with |d| (1024 + sc_k q_k) in place of
 *    |d| sc_k q_k, cA = 2^-17 on the matrix cores (groups of 128).  The
 *    prefill GEMM multiplies its f16 activations exactly (no first term).
 *    The method's bound |y - y_exact| <= 2e-4 A follows whenever
 *    sum_g max|w| S4_g <= 4 A and B <= 200 A (B <= 15 A on the matrix cores):
 *    weights spread within each group (a group whose weights sit only on its
 *    smallest activations is outside it) and factored terms that do not
 *    cancel.  Outliers of any size, up to four per group, with zero weights
 *    included, stay inside it.  An f16 output adds its rounding to nearest.
 *    Non-finite x gives NaN in every output of its token.  The statements
 *    assume no product or partial sum overflows or underflows f32.
 *  - Calls are stateless and may be made from several host threads.
 */
#ifndef Q4K_H
#define Q4K_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define Q4K_API __attribute__((visibility("default")))
#else
#define Q4K_API
#endif

/*
 * The two enums below also name the ends of the int range (the *_INT_MIN_ and
 * *_INT_MAX_ members, never returned or accepted as values): every int is
 * then a value of the type, also in C++, so a caller may pass any code and
 * an unknown one is rejected (Q4K_ERR_INVALID_ARG; "unknown status" from
 * q4k_status_string) rather than being out of the type's range.
 */
typedef enum {
    Q4K_OK = 0,
    Q4K_ERR_INVALID_ARG = 1,       /* null pointer, negative size, overlap, size overflow */
    Q4K_ERR_UNSUPPORTED_SHAPE = 2, /* k % 256 != 0, or a shape beyond a call's stated limits */
    Q4K_ERR_MISALIGNED = 3,        /* w not 16-B aligned, or x/y not 4-B aligned */
    Q4K_ERR_LAUNCH = 4,            /* the HIP runtime refused a launch */
    Q4K_STATUS_INT_MIN_ = -2147483647 - 1,
    Q4K_STATUS_INT_MAX_ = 2147483647
} q4k_status;

/* Element type of activations and outputs in the *_dt calls. */
typedef enum {
    Q4K_F32 = 0, /* IEEE binary32 */
    Q4K_F16 = 1, /* IEEE binary16: inputs widened exactly, outputs rounded to nearest even */
    Q4K_DTYPE_INT_MIN_ = -2147483647 - 1,
    Q4K_DTYPE_INT_MAX_ = 2147483647
} q4k_dtype;

/* Bytes of one Q4_K super-block and weights per super-block. */
#define Q4K_BLOCK_BYTES 144
#define Q4K_BLOCK_WEIGHTS 256

/* Bytes of one Q8_0 block and weights per block (an f16 scale, then 32
 * signed bytes). */
#define Q4K_Q8_0_BLOCK_BYTES 34
#define Q4K_Q8_0_BLOCK_WEIGHTS 32

/*
 * Batch-1 GEMV (the decode case: "@simulatte/doppler 0.1.7 -> 0.1.8",
 * matmul-selection.js, resolveMatmulPhase treats M == 1 as decode and
 * selectQ4KFusedVariant picks the fused Q4K variant for it).
 *   w : Q4_K matrix [n, k] (n*(k/256)*144 bytes)
 *   x : f32 [k]
 *   y : f32 [n], written: y[r] = sum_c W[r,c] x[c]
 */
Q4K_API q4k_status q4k_gemv(const void *w, const float *x, float *y, int64_t n, int64_t k, void *stream);

/*
 * Batch-1 GEMV with f16 or f32 activations and outputs ("@simulatte/doppler
 * 0.1.7 -> 0.1.8", matmul-selection.js: selectQ4KFusedVariant chooses the
 * fused Q4K kernel by aDtype and wantF16Output, and an f16 activation may
 * still produce an f32 output).  Computes what q4k_gemv computes on the
 * activations widened to f32; an f16 output is that f32 result rounded to
 * nearest even (beyond the f16 range: +-inf).
 *   x : [k] of x_dtype, aligned to its element size
 *   y : [n] of y_dtype, aligned to its element size
 * Other arguments, errors and aliasing rules as q4k_gemv; an unknown dtype is
 * Q4K_ERR_INVALID_ARG.
 */
Q4K_API q4k_status q4k_gemv_dt(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype,
                               int64_t n, int64_t k, void *stream);

/*
 * Batch-1 GEMV with a residual added in the same pass: y = W x + r (the
 * down projection of a decode step feeding the residual stream;
 * "qualia_core_db/inference/cuda_lane/mod.rs" re-exports
 * try_q4k_soa_ffn_block_residual from its gemv module).
 *   w : Q4_K matrix [n, k];  x : f32 [k];  r : f32 [n]
 *   y : f32 [n], written: y[i] = sum_c W[i,c] x[c] + r[i].
 * r may be y itself (an in-place residual add); otherwise r and y must not
 * overlap.  y must not overlap w or x.
 */
Q4K_API q4k_status q4k_gemv_residual(const void *w, const float *x, const float *r, float *y, int64_t n, int64_t k,
                                     void *stream);

/* One matrix of q4k_gemv_multi. */
typedef struct {
    const void *w;    /* Q4_K matrix [n, k], 16-byte aligned */
    float *y;         /* f32 [n] output (the q half, [n/2], with y_gate) */
    int64_t n;        /* rows (0: skipped) */
    float *y_gate;    /* NULL, or the gate half [n/2] of a per-head interleaved q projection */
    int64_t head_dim; /* with y_gate: rows per half head (a power of two dividing n/2) */
} q4k_gemv_item;

/* Largest number of matrices in one q4k_gemv_multi call. */
#define Q4K_MAX_MULTI 8

/*
 * Several batch-1 GEMVs with the same k against one x, in one launch where
 * k <= 4096 (the q, k and v projections of a decode step;
 * "qualia_core_db/inference/cuda_lane/mod.rs" re-exports try_q4k_soa_qkv
 * from its gemv module).  For each item: y[i] = sum_c W[i,c] x[c].
 *   items : host array of `count` items, 0 <= count <= Q4K_MAX_MULTI
 * No output may overlap another output, any weight matrix, or x.  Each
 * result equals what q4k_gemv gives for that matrix.
 *
 * An item with y_gate set has its output de-interleaved per head as it is
 * stored (the split of an attention-output-gate q projection, "@simulatte/
 * doppler 0.1.7 -> 0.1.8", kernels/split_qg: q_proj rows interleave each
 * head's q rows and gate rows).  With D = head_dim, row h*2D + j goes to
 * y[h*D + j] for j < D and to y_gate[h*D + j - D] otherwise; the values are
 * those q4k_gemv gives for the rows.  head_dim must be a power of two with
 * n % (2*head_dim) == 0 (else Q4K_ERR_INVALID_ARG), and k <= 4096 (else
 * Q4K_ERR_UNSUPPORTED_SHAPE).  Without y_gate, head_dim is ignored.
 */
Q4K_API q4k_status q4k_gemv_multi(const q4k_gemv_item *items, int count, const float *x, int64_t k, void *stream);

/*
 * Batch-1 GEMV over Q8_0 weights, the second block format of the decode path
 * ("qualia_core_db/inference/cuda_lane/mod.rs" re-exports try_q8_0_cuda_gemv,
 * q8_0_gemv_oracle_into, Q8_0_BLOCK_BYTES and Q8_0_BLOCK_ELEMS from its q8
 * module).  Each row of k weights is k/32 blocks of 34 bytes: d (IEEE
 * binary16, little-endian), then 32 signed bytes q; weight e of a block is
 * f32(d) * q[e] (the GGUF Q8_0 block).
 *   w : Q8_0 matrix [n, k] (n*(k/32)*34 bytes), 2-byte aligned
 *   x : f32 [k];  y : f32 [n], written: y[i] = sum_c W[i,c] x[c].
 * k % 32 != 0 -> Q4K_ERR_UNSUPPORTED_SHAPE.  Rows with an even number of
 * blocks in a 4-byte aligned matrix take the streaming kernels (fastest with
 * k % 256 == 0 in a 16-byte aligned matrix, k <= 4096 or 8192 < k <= 12288:
 * the weights then pass through LDS; the results are the same bits either
 * way); any other layout a slower one-wave-per-row kernel.  Accuracy as
 * q4k_gemv.
 */
Q4K_API q4k_status q4k_q8_0_gemv(const void *w, const float *x, float *y, int64_t n, int64_t k, void *stream);

/*
 * Skinny GEMM over the same weights for m tokens (selectQ4KFusedVariant's
 * non-M1 variant; "Module qwen3_attention" names a W4A16 batched path).
 *   x : f32 [m, k] row-major (token-major), y : f32 [m, n] row-major:
 *   y[t, r] = sum_c W[r,c] x[t,c].
 * A few tokens (2 <= m <= 4 with k <= 4096, and m == 2 with k <= 16384) run
 * on the streaming GEMV kernels, which decode each weight group once per
 * pair of tokens and need no scratch: every token's row is bit for bit what
 * q4k_gemv computes for that token.  The exception is 3 or 4 tokens with
 * k <= 4096 over n >= 64 * (compute units) rows, which the matrix cores do
 * faster.  Every other m >= 2 runs on the matrix cores (each weight decoded
 * once per 64 tokens).  There, with n >= 16 *
 * (compute units of the device), every output is summed in a fixed order, or
 * from exactly two partial sums (K halved between two workgroups: k == 4096
 * with at most 16 tokens, an f32 y and at most 8 16-row tiles per compute unit,
 * or k > 4096 with n == 16 * (compute units)) added into a zeroed y, whose
 * sum does not depend on their order: the call is bitwise
 * reproducible.  With fewer rows the K range is split across more workgroups
 * whose partial sums are added into y with f32 atomics, so the last bits may
 * differ between runs (every run is inside the error bound).  y is
 * overwritten, not accumulated.
 */
Q4K_API q4k_status q4k_gemv_batched(const void *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                            void *stream);

/*
 * q4k_gemv_batched with f16 or f32 activations and outputs (x [m, k] of
 * x_dtype, y [m, n] of y_dtype, each aligned to its element size): the
 * skinny-GEMM side of selectQ4KFusedVariant's aDtype / wantF16Output choice
 * ("@simulatte/doppler 0.1.7 -> 0.1.8", matmul-selection.js).  Computes what
 * q4k_gemv_batched computes on the activations widened to f32; f16 outputs
 * are rounded to nearest even.  With f16 activations, m >= 128 and a
 * 16-byte aligned x the call runs q4k_prefill_gemm instead (the kernel for
 * prefill sizes): the same bound and bitwise reproducible, but not bit for
 * bit the f32 path's result.  The scratch is that of q4k_gemv_batched,
 * plus 4*m*n bytes for an f16 output when K is split across workgroups (the
 * partial sums are added in f32 first).  Errors and aliasing as
 * q4k_gemv_batched; an unknown dtype is Q4K_ERR_INVALID_ARG.
 */
Q4K_API q4k_status q4k_gemv_batched_dt(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype,
                                       int64_t m, int64_t n, int64_t k, void *stream);

/*
 * q4k_gemv_batched_dt for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Computes exactly what q4k_gemv_batched_dt computes (the
 * same kernels, the same order of sums) and calls no allocator: the scratch
 * the call needs (q4k_gemv_batched_workspace_size) comes from one array of
 * Q4K_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on,
 * from its first such call until the process ends.  A call that needs more
 * is refused with Q4K_ERR_UNSUPPORTED_SHAPE and launches nothing (at k = 4096
 * up to 64 tokens need about 1.1 MB; prefill sizes with f16 activations can
 * exceed the array).  Every call on one GPU shares that GPU's array: calls on
 * one GPU whose work overlaps in time (on different streams without
 * ordering between them) race; calls ordered on one stream do not.  Its
 * contents are garbage before and after each call.  Errors and aliasing as
 * q4k_gemv_batched_dt.
 */
#define Q4K_NOALLOC_SCRATCH_BYTES (16 << 20)
Q4K_API q4k_status q4k_gemv_batched_noalloc(const void *w, const void *x, q4k_dtype x_dtype, void *y,
                                            q4k_dtype y_dtype, int64_t m, int64_t n, int64_t k, void *stream);

/*
 * Prefill-size GEMM with f16 activations (W4A16): the prefill side of
 * resolveMatmulPhase / selectQ4KFusedVariant ("@simulatte/doppler 0.1.7 ->
 * 0.1.8", matmul-selection.js), for hundreds of tokens at once.
 *   w : Q4_K matrix [n, k], 16-byte aligned
 *   x : f16 [m, k] token-major, 16-byte aligned
 *   y : [m, n] of y_dtype (f32 or f16), aligned to its element size:
 *       y[t, r] = sum_c W[r,c] x[t,c], computed from exact f16 operands on the
 *       matrix cores with f32 accumulation (the same bound as q4k_gemv);
 *       bitwise reproducible; an f16 y is the f32 result rounded to nearest
 *       even.
 * Any m >= 1 is accepted; the kernel works in 128-token tiles, so it is
 * meant for m >= 128 (q4k_gemv_batched_dt covers fewer tokens).  Takes
 * scratch (as described at the top) of 2*m'*k + 32*(m'/128)*(k/256)*128
 * bytes, m' = m rounded up to 128.
 * k > 2^24 -> Q4K_ERR_UNSUPPORTED_SHAPE.  Other errors and aliasing as
 * q4k_gemv_batched.
 */
Q4K_API q4k_status q4k_prefill_gemm(const void *w, const void *x, void *y, q4k_dtype y_dtype, int64_t m, int64_t n,
                                    int64_t k, void *stream);

/*
 * Caller-provided scratch for the two calls above that need any, so that the
 * library allocates nothing (a caller that keeps its own pool, or records the
 * calls into a HIP graph without allocation nodes).
 *
 * q4k_gemv_batched_workspace_size / q4k_prefill_workspace_size write to
 * *bytes the scratch that q4k_gemv_batched_dt / q4k_prefill_gemm need for
 * these dtypes and sizes on the CURRENT device (the split of K follows the
 * device's compute-unit count); 0 where none is needed (m <= 1, k == 0, an
 * empty call, the few-token sizes that q4k_gemv_batched runs on the
 * streaming kernels).  Same shape checks and status codes as the calls themselves;
 * bytes == NULL is Q4K_ERR_INVALID_ARG.  Nothing is enqueued.
 *
 * q4k_gemv_batched_ws / q4k_prefill_gemm_ws compute exactly what
 * q4k_gemv_batched_dt / q4k_prefill_gemm compute (the same kernels, the same
 * order of sums) with `workspace`, a device buffer of workspace_bytes owned by
 * the caller, in place of the library's scratch.  The workspace must
 * be 256-byte aligned (else Q4K_ERR_MISALIGNED), hold at least the queried
 * size (else Q4K_ERR_INVALID_ARG; it may be NULL when that size is 0) and
 * overlap none of w, x, y (Q4K_ERR_INVALID_ARG).  Its contents are garbage before and after
 * the call; the call uses it until the stream reaches the end of the call's
 * work, so calls in flight at the same time need separate workspaces.
 */
Q4K_API q4k_status q4k_gemv_batched_workspace_size(q4k_dtype x_dtype, q4k_dtype y_dtype, int64_t m, int64_t n,
                                                   int64_t k, int64_t *bytes);
Q4K_API q4k_status q4k_gemv_batched_ws(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype,
                                       int64_t m, int64_t n, int64_t k, void *workspace, int64_t workspace_bytes,
                                       void *stream);
Q4K_API q4k_status q4k_prefill_workspace_size(q4k_dtype y_dtype, int64_t m, int64_t n, int64_t k, int64_t *bytes);
Q4K_API q4k_status q4k_prefill_gemm_ws(const void *w, const void *x, void *y, q4k_dtype y_dtype, int64_t m, int64_t n,
                                       int64_t k, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Fused gate/up GEMV with SwiGLU ("qualia_core_db/inference/cuda_lane/mod.rs",
 * try_q4k_soa_fused_swiglu; "Struct WgslForwardPass", silu_mul_shader):
 *   w_gate, w_up : two separate Q4_K matrices [n, k]
 *   x : f32 [k]; h : f32 [n], written: h[r] = silu(g[r]) * u[r] with
 *   g = W_gate x, u = W_up x, silu(t) = t / (1 + exp(-t)).
 */
Q4K_API q4k_status q4k_fused_swiglu(const void *w_gate, const void *w_up, const float *x, float *h, int64_t n,
                            int64_t k, void *stream);

/*
 * Dequantize to dense f32 (the "dequantize once to dense f32" fallback of the
 * cuda_lane module docs), bit-exact: out[r, c] = f32(f32(d*sc)*q - f32(dmin*m)).
 *   out : f32 [n, k] row-major.
 */
Q4K_API q4k_status q4k_dequant(const void *w, float *out, int64_t n, int64_t k, void *stream);

/*
 * Static, NUL-terminated description of a status code (never NULL; codes the
 * library does not define give "unknown status").  No page defines this
 * call: it is the C form of the fallible entry points of the cuda_lane module
 * docs (try_q4k_soa_gemv and its siblings return an error value that a
 * caller can print), which this ABI's status codes stand for.
 */
Q4K_API const char *q4k_status_string(q4k_status s);

/* ABI version of this header (major*100 + minor); q4k_abi_version() of the
 * library it was built with returns the same number. */
#define Q4K_ABI_VERSION 109
Q4K_API int q4k_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */
