/*
 * sp24.h -- C ABI of libsp24.so: 2:4 semi-structured sparsity on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (sources: "2:4 Structured Sparsity Explained", sections "How
 * 2:4 sparsity works" and "How to make a model 2:4 sparse"; "Production 2:4
 * Structured Sparsity for LLMs", sections "From Unstructured Pruning to
 * Hardware-Accelerable Sparsity" and "Sparse Tactic Audit"; the
 * 2:4-versus-quantization paper, section 2 "Sparse tensor cores" and
 * section 3.5 "Measuring speed"):
 *
 *   - a 2:4 operand keeps, in every group of 4 consecutive elements along the
 *     reduction axis K, the 2 elements of largest magnitude (ties: the lower
 *     index wins) and stores them in half the space, plus a 2-bit position
 *     (0..3) for each kept value;
 *   - a sparse MMA multiplies that compressed first operand by a dense second
 *     operand, the positions selecting the matching dense elements, for up
 *     to twice the dense rate;
 *   - a dense GEMM runs on the same shapes, and a per-shape tactic keeps
 *     whichever is faster, falling back to dense when sparse is not.
 *
 * Conventions shared by every call
 *   - All tensors are row-major with K contiguous.  W is (N, K), X is (M, K),
 *     Y = X * W^T is (M, N).  "rows" of a compressed operand is N for W and M
 *     for X.
 *   - Compressed form of a rows x K operand:
 *       values : rows x K/2 elements of the operand's dtype, row stride K/2.
 *                Group g of row r stores its two kept elements at
 *                values[r][2g] (lower position p0) and values[r][2g+1]
 *                (higher position p1), bit-for-bit copies of the input.
 *       meta   : rows x ceil(K/32) uint32 words, row stride ceil(K/32).
 *                Group g is the nibble p0 | p1 << 2 (p0 < p1) at bits
 *                4*(g%8) .. 4*(g%8)+3 of meta[r][g/8]; nibbles past the last
 *                group of a row are 0.  Only the six nibbles 0x4, 0x8, 0xC,
 *                0x9, 0xD, 0xE occur.
 *   - Magnitude is the integer value of the sign-stripped bit pattern; +0
 *     and -0 tie, NaN ranks above Inf.  Dropped positions decompress to +0.
 *   - fp8 is OCP E4M3 (e4m3fn).  A GEMM takes an optional fp32 scale per row
 *     of X (per token) and per row of W (per output channel), NULL meaning 1:
 *     Y[m][n] = (sum_k x[m][k] * w[n][k]) * scale_x[m] * scale_w[n]
 *     (one fp32 scale per row of X and per output channel of W, as the
 *     2:4-versus-quantization paper's section 2 "Quantization" sets fp8 up).
 *   - Accumulation is fp32; the output is rounded once, to nearest even.
 *   - Every pointer argument is a device pointer unless marked "host".  The
 *     caller allocates and owns every buffer; the library keeps no device
 *     memory and holds no global mutable state (calls are thread-safe).
 *   - Every call validates its arguments on the host before any HIP call and
 *     returns an sp24_status without touching the device on failure.  Work
 *     is enqueued asynchronously on `stream` (0 = the null stream); only
 *     sp24_select_tactic synchronizes.  Device faults surface at the
 *     caller's next synchronization.  No C++ exception crosses this ABI.
 */
#ifndef SP24_H
#define SP24_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SP24_F16 = 0,   /* IEEE binary16 */
    SP24_BF16 = 1,  /* bfloat16 */
    SP24_E4M3 = 2,  /* OCP FP8 E4M3 (e4m3fn) */
    SP24_F32 = 3,   /* binary32: an output dtype only */
    SP24_I8 = 4     /* two's complement int8 (quantized, with per-row scales) */
} sp24_dtype;

typedef enum {
    SP24_SPARSE_W = 0, /* the weight W (N, K) is the compressed operand (static weights) */
    SP24_SPARSE_X = 1  /* the activation X (M, K) is the compressed operand (dynamic) */
} sp24_operand;

typedef enum {
    SP24_OK = 0,
    SP24_E_NULL = 1,     /* a required pointer is NULL */
    SP24_E_SHAPE = 2,    /* a size is negative, K % 4 != 0, a leading dimension < K, or a GEMM
                            operand (plus 256 rows) of 2 GiB or more */
    SP24_E_DTYPE = 3,    /* unsupported dtype or dtype combination */
    SP24_E_ALIGN = 4,    /* pointer not 16-byte aligned, or K not a multiple of the GEMM's K tile */
    SP24_E_HIP = 5       /* the HIP runtime reported an error (launch, event, device query) */
} sp24_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *sp24_status_str(sp24_status s);

/* Library version string, e.g. "sp24 0.1.0 gfx950" (static storage). */
const char *sp24_version(void);

/* Words of metadata per row: ceil(K / 32). */
int64_t sp24_meta_words_per_row(int64_t K);

/*
 * Prune + compress ("2:4 Structured Sparsity Explained", "How to make a model
 * 2:4 sparse": keep the two largest magnitudes of each group of four; and
 * "How 2:4 sparsity works": half-size values plus a 2-bit index per kept
 * value).  One pass: the dense operand is read once, values and meta are
 * written once (the fused form of the paper's section 3.5).
 *   dt      SP24_F16, SP24_BF16, SP24_E4M3 or SP24_I8 (for int8 the magnitude
 *           is |x|, so -128 ranks above 127)
 *   rows, K dense operand is rows x K; K % 4 == 0; rows, K >= 0 (0 is a no-op)
 *   src     rows x K, row stride ld_src elements (ld_src >= K)
 *   values  out: rows x K/2 elements (dt), row stride K/2
 *   meta    out: rows x ceil(K/32) uint32, row stride ceil(K/32)
 * Misaligned pointers or strides are accepted (a slower kernel runs).
 */
sp24_status sp24_prune_compress(sp24_dtype dt, int64_t rows, int64_t K,
                                const void *src, int64_t ld_src,
                                void *values, uint32_t *meta, hipStream_t stream);

/*
 * Decompress: the inverse of sp24_prune_compress ("Production 2:4 Structured
 * Sparsity for LLMs", playbook step 2: the dense view has exactly two zeros
 * in every four along the reduction axis).  Every position of dst is
 * written: +0 where a group dropped an element, the kept value (bit copy)
 * elsewhere.  For an illegal nibble (p0 >= p1, never produced by
 * sp24_prune_compress) value 0 is written at p0 and then value 1 at p1.
 *   dst     out: rows x K, row stride ld_dst elements (ld_dst >= K)
 */
sp24_status sp24_decompress(sp24_dtype dt, int64_t rows, int64_t K,
                            const void *values, const uint32_t *meta,
                            void *dst, int64_t ld_dst, hipStream_t stream);

/*
 * The fused online fp8 path for a dynamic operand (the 2:4-versus-quantization
 * paper, sections 3.5 "Measuring speed" and 4.2 "Speed": quantize, prune and
 * compress in one pass that reads the operand once and writes the kept values
 * and their indices once; section 2 "Quantization": one scale per row).
 * Per row r of the f16 / bf16 source:
 *   scales[r] = max|x| / 448 in fp32 (1 for an all-zero row);
 *   codes     = e4m3fn(x / scales[r]), the quotient in fp32, rounded to
 *               nearest even and saturated at 448;
 *   then the magnitude 2:4 prune and compress of the codes, exactly as
 *   sp24_prune_compress does for SP24_E4M3 input.
 *   src_dt    SP24_F16 or SP24_BF16
 *   rows, K   0 <= rows <= 2^24 (else SP24_E_SHAPE);
 *             K % 32 == 0 (whole metadata words), else SP24_E_ALIGN
 *   src       rows x K, row stride ld_src elements (ld_src >= K, ld_src % 8 == 0)
 *   values    out: rows x K/2 e4m3 bytes;  meta  out: rows x K/32 words
 *   scales    out: rows fp32
 *   Pointers 16-byte aligned (scales 4-byte).  The outputs feed
 *   sp24_gemm(SP24_SPARSE_X, SP24_E4M3, ..., scale_x = scales, ...).
 */
sp24_status sp24_quantize_prune_compress(sp24_dtype src_dt, int64_t rows, int64_t K,
                                         const void *src, int64_t ld_src,
                                         void *values, uint32_t *meta, float *scales,
                                         hipStream_t stream);

/*
 * The same per-row e4m3 quantization without the prune: every code, rows x K
 * e4m3 bytes into `dst` (row stride K), one fp32 scale per row.  The dense
 * side of the online fp8 comparison: each side pays for producing its own
 * input.  Same dtypes, sizes, alignment and errors as above.
 */
sp24_status sp24_quantize_e4m3(sp24_dtype src_dt, int64_t rows, int64_t K,
                               const void *src, int64_t ld_src, void *dst, float *scales,
                               hipStream_t stream);

/*
 * The fused online int8 path: the same one-pass quantize, prune and compress
 * with symmetric int8 codes (the 2:4-versus-quantization paper, section 4.2
 * "Speed": 2:4 with INT8; section 2 "Quantization": one scale per row).
 * Per row r of the f16 / bf16 source:
 *   scales[r] = max|x| / 127 in fp32 (1 for an all-zero row; a NaN does not
 *               count toward the maximum);
 *   codes     = x / scales[r] in fp32 (correctly rounded), rounded to the
 *               nearest integer (ties to even) and saturated to [-127, 127];
 *               a NaN quotient codes to 0, so -128 never occurs;
 *   then the magnitude 2:4 prune and compress of the codes, exactly as
 *   sp24_prune_compress does for SP24_I8 input.
 *   Dtypes, sizes, strides, alignment and errors as sp24_quantize_prune_compress;
 *   values out: rows x K/2 int8;  meta out: rows x K/32 words;  scales out: rows
 *   fp32.  The outputs feed sp24_gemm(SP24_SPARSE_X, SP24_I8, ..., scale_x =
 *   scales, ...).
 */
sp24_status sp24_quantize_i8_prune_compress(sp24_dtype src_dt, int64_t rows, int64_t K,
                                            const void *src, int64_t ld_src,
                                            void *values, uint32_t *meta, float *scales,
                                            hipStream_t stream);

/*
 * The same per-row int8 quantization without the prune: every code, rows x K
 * int8 into `dst` (row stride K), one fp32 scale per row -- the dense int8
 * GEMM's input on the online int8 comparison.  Same dtypes, sizes, alignment
 * and errors as above.
 */
sp24_status sp24_quantize_i8(sp24_dtype src_dt, int64_t rows, int64_t K,
                             const void *src, int64_t ld_src, void *dst, float *scales,
                             hipStream_t stream);

/*
 * Sparse x dense GEMM, Y = X * W^T (the paper's section 2 "Sparse tensor
 * cores": the compressed first operand and its indices select the matching
 * elements of the dense operand).
 *   which     SP24_SPARSE_W: (values, meta) is W (N x K) compressed and
 *             `dense` is X (M x K).  SP24_SPARSE_X: (values, meta) is X
 *             compressed and `dense` is W.
 *   in_dt     SP24_F16, SP24_BF16, SP24_E4M3 or SP24_I8 (both operands; int8
 *             products accumulate exactly in int32, converted to fp32 before
 *             the scales: the 2:4 + INT8 variant of the 2:4-versus-
 *             quantization paper, section 4.2 "Speed")
 *   out_dt    SP24_F16 or SP24_BF16 or SP24_F32 for 16-bit inputs;
 *             SP24_BF16 or SP24_F32 for SP24_E4M3 and SP24_I8
 *   M, N, K   M, N >= 0; K % 64 == 0 (16-bit) or K % 128 == 0 (8-bit), else
 *             SP24_E_ALIGN: the shape is not eligible and the caller runs
 *             dense_gemm instead (a visible fallback, never a silent one)
 *   scale_x   M fp32 per-token scales, or NULL (= 1); used with 8-bit inputs
 *   scale_w   N fp32 per-channel scales, or NULL (= 1); used with 8-bit inputs
 *   Y         out: M x N of out_dt, row stride N
 *   All pointers 16-byte aligned.
 */
sp24_status sp24_gemm(sp24_operand which, sp24_dtype in_dt, sp24_dtype out_dt,
                      int64_t M, int64_t N, int64_t K,
                      const void *values, const uint32_t *meta, const void *dense,
                      const float *scale_x, const float *scale_w,
                      void *Y, hipStream_t stream);

/*
 * Dense GEMM on the same shapes, Y = X * W^T: the baseline every sparse
 * tactic is timed against and the target of every fallback ("Production
 * 2:4 Structured Sparsity for LLMs", section "Dense Fallback and Hybrid
 * Sparsity Design").  Same dtypes, scales and layout as sp24_gemm.  It
 * accepts every K that fills whole 16-byte chunks of a row, K % 8 == 0
 * (16-bit) or K % 16 == 0 (fp8), so that it can take the shapes the sparse
 * path rejects; else SP24_E_ALIGN.  Pointers 16-byte aligned.
 */
sp24_status dense_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K,
                       const void *X, const void *W,
                       const float *scale_x, const float *scale_w,
                       void *Y, hipStream_t stream);

/*
 * Hybrid sparse + dense GEMM in one launch ("Production 2:4 Structured
 * Sparsity for LLMs", section "Dense Fallback and Hybrid Sparsity Design":
 * dense regions kept next to 2:4 regions of one weight, as SpenseGPT does).
 * The weight's output channels are split by row: the first N_s rows are
 * 2:4-compressed, the next N_d rows stay dense, and the outputs are disjoint:
 *   Y[m][n]       = sum_k X[m][k] * Ws[n][k]          n <  N_s
 *   Y[m][N_s + n] = sum_k X[m][k] * Wd[n][k]          n <  N_d
 * (times scale_x[m] * scale_w[column] for fp8).  The caller chooses which
 * rows go where and orders them so (any row permutation of W permutes the
 * columns of Y alike).  One kernel runs both regions: its dense tiles feed
 * the same sparse instruction twice per group of four, once with positions
 * (0, 1) and once with (2, 3), so both regions share the pipeline and the
 * epilogue and no region waits for the other.
 *   in_dt, out_dt  as sp24_gemm
 *   M, N_s, N_d, K M, N_s, N_d >= 0; K % 64 (16-bit) or K % 128 (fp8), else
 *                  SP24_E_ALIGN; N_s % 8 == 0 (the dense outputs start on a
 *                  16-byte boundary), else SP24_E_ALIGN
 *   values, meta   Ws compressed: N_s x K/2 values, N_s x K/32 words
 *   W_d            N_d x K dense, row-major
 *   X              M x K dense, row-major
 *   scale_x        M floats or NULL;  scale_w  N_s + N_d floats or NULL
 *   Y              M x (N_s + N_d) of out_dt, row-major
 * Same sizes limits, alignment and errors as sp24_gemm; values/meta may be
 * NULL when N_s == 0 and W_d when N_d == 0.
 */
sp24_status sp24_hybrid_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N_s, int64_t N_d,
                             int64_t K, const void *values, const uint32_t *meta, const void *W_d,
                             const void *X, const float *scale_x, const float *scale_w, void *Y,
                             hipStream_t stream);

/* The name of the kernel sp24_hybrid_gemm launches for this shape, as
 * sp24_gemm_kernel does for the plain GEMMs (host only; NULL if rejected). */
const char *sp24_hybrid_kernel(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N_s,
                               int64_t N_d, int64_t K);

/*
 * Hybrid sparse + dense GEMM split along K, in one launch ("Production 2:4
 * Structured Sparsity for LLMs", section "Dense Fallback and Hybrid Sparsity
 * Design"; the SlideSparse page, Spense abstract: each weight matrix split
 * into a 2:4 region and a dense region).  Columns [0, K_s) of every weight
 * row are 2:4-compressed, columns [K_s, K) stay dense, and both ranges add
 * into the same outputs:
 *   Y[m][n] = sum_{k < K_s} X[m][k] * Ws[n][k] + sum_{k >= K_s} X[m][k] * Wd[n][k - K_s]
 * (times scale_x[m] * scale_w[n] for 8-bit inputs), accumulated in one fp32
 * (int32 for int8) accumulator per output and rounded once.  The caller
 * chooses which columns go where (a permutation of K applied to the columns
 * of both W and X leaves Y unchanged).  Each workgroup runs the 2:4 range of
 * its tile on the sparse instruction and then the dense range on the dense
 * one, into the same registers.
 *   in_dt, out_dt  as sp24_gemm
 *   M, N, K_s, K   M, N >= 0; 0 <= K_s <= K, else SP24_E_SHAPE; K % 64
 *                  (16-bit) or K % 128 (8-bit), and K_s % 256, else
 *                  SP24_E_ALIGN
 *   values, meta   Ws compressed: N x K_s/2 values, N x K_s/32 words
 *   W_d            N x (K - K_s) dense, row-major (row stride K - K_s)
 *   X              M x K dense, row-major
 *   scale_x        M floats or NULL;  scale_w  N floats or NULL
 *   Y              M x N of out_dt, row-major
 * Same size limits, alignment and errors as sp24_gemm; values/meta may be
 * NULL when K_s == 0 and W_d when K_s == K.
 */
sp24_status sp24_ksplit_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K_s,
                             int64_t K, const void *values, const uint32_t *meta, const void *W_d,
                             const void *X, const float *scale_x, const float *scale_w, void *Y,
                             hipStream_t stream);

/* The name of the kernel sp24_ksplit_gemm launches for this shape (host
 * only; NULL if rejected). */
const char *sp24_ksplit_kernel(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N,
                               int64_t K_s, int64_t K);

/*
 * The name of the kernel that sp24_gemm (sparse != 0) or dense_gemm
 * (sparse == 0) launches for this shape and dtype, without launching
 * anything: a pure host function, no HIP call.  The same names appear in
 * sp24_tactic.kernel and, as template instantiations, in profiler traces.
 * Returns NULL when the call would be rejected on its dtypes or shape
 * (including SP24_E_ALIGN on K), "none" when M or N is 0 and "fill_zero"
 * when K is 0.  The returned string is static; do not free it.
 */
const char *sp24_gemm_kernel(int sparse, sp24_operand which, sp24_dtype in_dt,
                             sp24_dtype out_dt, int64_t M, int64_t N, int64_t K);

/* Per-shape tactic record ("Production 2:4 Structured Sparsity for LLMs",
 * section "Sparse Tactic Audit": eligible / selected / reason per layer). */
typedef struct {
    int eligible;          /* 1 if the sparse path accepts this shape and dtype */
    int selected;          /* 1 = sparse, 0 = dense */
    double t_sparse_us;    /* median device time of the sparse GEMM */
    double t_compress_us;  /* median device time of prune+compress (SP24_SPARSE_X only, else 0) */
    double t_dense_us;     /* median device time of the dense GEMM */
    double ratio;          /* t_dense / median(t_compress + t_sparse per rep); > 1: sparse faster */
    char reason[96];       /* why the choice was made, e.g. "Dense kernel 1.15x faster" */
    char kernel[64];       /* name of the kernel that the chosen path actually launches */
} sp24_tactic;

/*
 * Times the sparse path (for SP24_SPARSE_X: prune+compress of X, then the
 * sparse GEMM; each side pays for producing its own input) against the dense
 * path on the caller's buffers and chooses sparse iff its median time is
 * strictly lower ("Production 2:4 Structured Sparsity for LLMs", section
 * "Sparse Tactic Audit": latency is the sole criterion; a dense kernel that
 * runs faster is chosen).
 *   values, meta   compressed operand (SP24_SPARSE_W), or scratch of the
 *                  compressed size that the timed compress overwrites
 *                  (SP24_SPARSE_X)
 *   dense_other    the operand that stays dense in the sparse path
 *   dense_pruned   the dense (pruned) form of the sparse operand, used by the
 *                  dense path (for SP24_SPARSE_X: the dense X that is
 *                  compressed on every sparse call)
 *   Y_scratch      M x N of out_dt, overwritten
 *   warmup, reps   untimed and timed repetitions of each path (reps >= 1)
 *   out            host: the record
 * An ineligible shape or dtype yields SP24_OK with eligible = 0, selected = 0,
 * reason "Alignment failure" or "Unsupported dtype", and only the dense path
 * timed.  Synchronizes `stream`.
 */
sp24_status sp24_select_tactic(sp24_operand which, sp24_dtype in_dt, sp24_dtype out_dt,
                               int64_t M, int64_t N, int64_t K,
                               const void *values, const uint32_t *meta,
                               const void *dense_other, const void *dense_pruned,
                               const float *scale_x, const float *scale_w, void *Y_scratch,
                               int warmup, int reps, hipStream_t stream, sp24_tactic *out);

/*
 * The decision rule alone, on host arrays of per-repetition times in
 * microseconds (a pure host function: no HIP call).  t_sparse holds
 * sparse(+compress) times, t_dense dense times; ns, nd >= 1 when eligible.
 * Fills selected, t_sparse_us (median), t_dense_us (median), ratio and
 * reason; leaves kernel and t_compress_us untouched.
 */
sp24_status sp24_tactic_decide(int eligible, const double *t_sparse, int ns,
                               const double *t_dense, int nd, sp24_tactic *out);

/*
 * Layer-level audit ("Production 2:4 Structured Sparsity for LLMs", section
 * "Audit Artifacts and Key Metrics", and step 3 of the playbook, "Run Tactic
 * Auditing and Profiling"): the counts, ratios and Sparse GPU-Time Coverage
 * of a model's manifest, aggregated from per-shape tactic records.
 *   records        n_records tactic records, one per distinct layer shape
 *   layer_counts   how many of the model's layers share each record (>= 0)
 *   other_time_us  GPU time of everything outside these layers (attention,
 *                  norms, ...), >= 0; 0 counts the audited layers alone
 *   out            host: the metrics
 * A layer's time is that of its selected path: t_sparse_us + t_compress_us
 * when it runs sparse (the compress term is 0 for a compressed weight), else
 * t_dense_us.  Every layer that does not run sparse is a dense fallback,
 * ineligible ones included.  Ratios with a zero denominator are 0.
 * A pure host function (no HIP call).  SP24_E_NULL for a missing pointer
 * (records and layer_counts may be NULL when n_records == 0); SP24_E_SHAPE
 * for n_records < 0, a negative count, or a negative or non-finite time.
 */
typedef struct {
    int64_t candidate_layers;         /* every audited layer */
    int64_t eligible_layers;          /* layers whose shape and dtype the sparse path accepts */
    int64_t sparse_selected_layers;   /* layers that run sparse */
    int64_t dense_fallback_layers;    /* candidate - sparse selected */
    double eligibility_ratio;         /* eligible / candidate */
    double sparse_selection_ratio;    /* sparse selected / eligible */
    double sparse_gpu_time_us;        /* sum of the time of the layers that run sparse */
    double total_gpu_time_us;         /* sum of every layer's selected time, + other_time_us */
    double sparse_gpu_time_coverage;  /* sparse_gpu_time_us / total_gpu_time_us */
} sp24_audit_metrics;

sp24_status sp24_audit_aggregate(const sp24_tactic *records, const int64_t *layer_counts,
                                 int64_t n_records, double other_time_us,
                                 sp24_audit_metrics *out);

#ifdef __cplusplus
}
#endif

#endif /* SP24_H */
