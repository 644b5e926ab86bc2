/*
 * mkp.h - run-time polymerized dense GEMM for AMD MI355X (gfx950).
 *
 * C = A . B with (M, N, K) known only at run time.  A fixed library of
 * hand-written CDNA4 micro-kernels (fixed uM x uN x uK tiles on bf16 MFMA with
 * fp32 accumulation) is composed per shape by a cost-model polymerizer
 * (MikPoly page, section 3: two-stage flow, micro-kernel performance model,
 * polymerization patterns and cost model); plans are cached by shape.
 *
 * Data types: A and B hold bf16 values (the upper 16 bits of an IEEE binary32,
 * passed as 16-bit words); C is IEEE binary32.  All matrices are row-major;
 * leading dimensions and strides count elements, not bytes.  Products are
 * accumulated in binary32.  C is overwritten (C := A.B, no alpha/beta): the
 * page's loops zero C before accumulating.
 *
 * Pointers A, B, C are device pointers owned by the caller; `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).  Calls are
 * asynchronous: they return once the work is enqueued.  Argument errors are
 * reported synchronously, before anything is written to C.  Faults inside a
 * kernel surface at the caller's next synchronisation of `stream`.
 *
 * Thread safety: every entry point may be called from several host threads,
 * on the same stream or on different ones.  The plan cache is shared under
 * a lock (a search on a miss runs outside it, so lookups of other shapes do
 * not wait); split-K workspaces are kept per (device, stream), and a call
 * holds its stream's workspace from the moment it takes it until its last
 * launch is enqueued, so calls on one stream from several threads run one
 * after the other on that stream without sharing partial results.  Two
 * calls that run concurrently on different streams must not write the same
 * C.  C must not alias A or B.  mkp_cache_clear() waits for the calls that
 * hold workspaces and then for the device before freeing them.
 *
 * Status codes: MKP_OK (0) on success, negative on error; mkp_last_error()
 * returns a thread-local message for the last error raised on this thread.
 */
#ifndef MKP_H
#define MKP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MKP_OK = 0,
    MKP_ERR_INVALID_ARG = -1, /* bad dimension, leading dimension, null pointer */
    MKP_ERR_UNSUPPORTED = -2, /* forced kernel/option the library cannot serve */
    MKP_ERR_OOM = -3,         /* split-K workspace could not be allocated */
    MKP_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    MKP_ERR_BUFFER = -5       /* output text buffer too small */
};

/* b_layout of mkp_gemm_ex */
enum {
    MKP_B_KN = 0,             /* B is K x N, ldb >= N */
    MKP_B_NK = 1              /* B is N x K, ldb >= K: C = A . B^T of the stored matrix */
};

/* activations of mkp_gemm_ex's epilogue */
enum {
    MKP_ACT_NONE = 0,
    MKP_ACT_RELU = 1,         /* max(x, 0) */
    MKP_ACT_GELU = 2,         /* x * Phi(x), Phi the standard normal distribution (erf form) */
    MKP_ACT_GELU_TANH = 3,    /* x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))) */
    MKP_ACT_SILU = 4          /* x * sigmoid(x) */
};

/* flags of mkp_plan_describe (align_flags) and mkp_plan_with_table (flags) */
enum {
    MKP_PLAN_EXHAUSTIVE = 1,  /* mkp_plan_with_table: score every candidate */
    MKP_PLAN_B_NK = 8         /* plan for B given as N x K (mkp_gemm_bt) */
};

/*
 * C[M x N] := A[M x K] . B[K x N].
 *   lda >= K, ldb >= N, ldc >= N (elements).  A, B, C may be NULL only when
 *   the matrix they name is empty.  M == 0 or N == 0: nothing is launched.
 *   K == 0: C := 0 (empty sum).  Pointers and leading dimensions need no
 *   particular alignment; unaligned ones are served by element-wise loads.
 * Source of the operation: MikPoly page, part 1 item 2 (C[i][j] += A[i][k] *
 * B[k][j] over zeroed C) and section 4 (tensor start addresses and loop trip
 * counts passed at run time to fixed-size micro-kernels).
 */
int mkp_gemm(int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda,
             const void *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/*
 * batch independent products C_b := A_b . B_b, entry b at A + b*strideA,
 * B + b*strideB, C + b*strideC (elements).  One plan serves every entry:
 * same-shape GEMMs merged into one batched GEMM (BladeDISC v0.2.0 release
 * notes, "GEMM merge" optimisation, second kind).  batch == 0 is a no-op.
 * The C_b must not overlap: |strideC| >= (M-1)*ldc + N unless batch == 1.
 */
int mkp_gemm_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, int64_t strideA,
                     const void *B, int64_t ldb, int64_t strideB,
                     float *C, int64_t ldc, int64_t strideC,
                     void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as mkp_gemm_batched -- same arguments, layout, result and errors --
 * that never allocates.  Its split-K partials and staging copies live in a
 * fixed device array inside the library, mkp_noalloc_scratch_bytes() bytes
 * (64 MiB) on every GPU the library runs on, held until the process ends.
 * A plan whose scratch would not fit is replaced by one with fewer K splits
 * and no staging copies (at the last resort no split at all, which needs
 * none), so every shape runs; split-K partials are always summed by a
 * second pass.  The array keeps the last call's contents between calls.
 * All calls on one GPU share that one array: calls that overlap on one GPU
 * (concurrent streams, or several host threads) race and may corrupt each
 * other's results -- issue them on one stream, one after the other.
 */
int mkp_gemm_batched_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda, int64_t strideA,
                             const void *B, int64_t ldb, int64_t strideB,
                             float *C, int64_t ldc, int64_t strideC,
                             void *stream);

/* Size in bytes of mkp_gemm_batched_noalloc's per-GPU scratch array. */
size_t mkp_noalloc_scratch_bytes(void);

/*
 * C[M x N] := A[M x K] . B^T with B given as N x K (row n holds the K values
 * of output column n; ldb >= K), the layout in which a linear layer keeps
 * its weights and attention keeps K.  Otherwise as mkp_gemm: same C, errors
 * (ldb < K is MKP_ERR_INVALID_ARG), alignment freedom and stream semantics.
 * The polymerizer composes it from the library's N x K micro-kernels (names
 * ending in "_nk"), whose B fragments come from LDS like A's.  Source: the
 * MikPoly page's GEMM (part 1 item 2) with B read through its transpose; the
 * layout is the workloads' (Korch page's and BladeDISC page's linear and
 * attention layers).
 */
int mkp_gemm_bt(int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda,
                const void *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream);

/* Batched mkp_gemm_bt: entry b at A + b*strideA, B + b*strideB (N x K),
 * C + b*strideC; as mkp_gemm_batched otherwise. */
int mkp_gemm_batched_bt(int64_t batch, int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda, int64_t strideA,
                        const void *B, int64_t ldb, int64_t strideB,
                        float *C, int64_t ldc, int64_t strideC,
                        void *stream);

/*
 * General form with a fused epilogue (Bolt page, epilogue fusion; its
 * persistent-kernel section writes the GEMM as D = alpha.A.W + beta.C):
 *   C_b := act(alpha * A_b . op(B_b) + beta * C_b + bias)   for b < batch,
 * op(B) = B for b_layout MKP_B_KN (B_b K x N), B^T for MKP_B_NK (B_b N x K).
 * bias: N fp32 values (device memory) added to every row, or NULL.  act: one
 * of MKP_ACT_*.  C is read only when beta != 0 (then it must hold values).
 * The epilogue runs where the final value is made -- in the micro-kernel's
 * store, or in the split-K reduction -- so it adds no pass over C.  With
 * alpha = 1, beta = 0, bias = NULL and MKP_ACT_NONE this is mkp_gemm_batched
 * (or _bt).  K == 0: C := act(beta * C + bias).  Batch strides as in
 * mkp_gemm_batched (ignored when batch == 1).  Errors as for mkp_gemm, plus
 * an unknown b_layout or act, or a non-finite alpha or beta.
 */
int mkp_gemm_ex(int64_t batch, int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda, int64_t strideA,
                const void *B, int64_t ldb, int64_t strideB, int b_layout,
                float *C, int64_t ldc, int64_t strideC,
                float alpha, float beta, const float *bias, int act,
                void *stream);

/*
 * Convolution as an implicit GEMM (the MikPoly page runs convolutions as
 * GEMMs on the same micro-kernels): y = act(conv2d(x, w) + bias), with
 *   x: N x H x W x C bf16 input (NHWC, contiguous),
 *   w: K x R x S x C bf16 filters (KRSC, contiguous: the K x (R S C) matrix
 *      of the GEMM's B, stored N x K),
 *   y: N x P x Q x K fp32 output (NPQK, contiguous),
 *   P = (H + 2 pad_h - dil_h (R - 1) - 1) / stride_h + 1, Q likewise;
 *   y[n][p][q][k] = sum over r, s, c of
 *     x[n][p stride_h - pad_h + r dil_h][q stride_w - pad_w + s dil_w][c] * w[k][r][s][c]
 *   (input outside the image reads as zero).
 * The GEMM is M = N P Q rows, N = K columns and K = R S C depth; it is
 * planned like mkp_gemm_bt and runs on the convolution form of the chosen
 * N x K micro-kernels, whose A loader gathers input rows (a K step of
 * channels within one filter tap when C is a multiple of 64 -- direct loads,
 * padding read from a zero page -- else 8 channels, or one element, at a
 * time; a 1 x 1 convolution with stride 1 and no padding is the plain GEMM
 * of the input as an (N H W) x C matrix).  bias: K fp32 values or NULL;
 * act: an MKP_ACT_* code.  Errors: bad
 * extents or a filter larger than the padded input (MKP_ERR_INVALID_ARG),
 * before anything is written; N == 0 or K == 0: nothing is launched.
 */
int mkp_conv2d(int64_t N, int64_t H, int64_t W, int64_t C,
               int64_t K, int64_t R, int64_t S,
               int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
               int64_t dil_h, int64_t dil_w,
               const void *x, const void *w, float *y,
               const float *bias, int act, void *stream);

/*
 * Grouped call: C_g[M x N_g] := A[M x K] . B_g for g < groups (1..4), the
 * products sharing A -- the merge of GEMMs that share an operand into one
 * product with the other operands side by side (BladeDISC page, GEMM merge,
 * first kind; e.g. the query, key and value projections of one input).  N, B, ldb, C, ldc are host arrays of
 * `groups` entries; B_g is K x N_g (ldb_g >= N_g).  One launch serves every
 * group: its tile columns are dealt group after group, so the widths need
 * not be tile multiples; the plan (one kernel and split factor over all
 * groups' tiles) is cached by M, K and the widths.  Groups with N_g == 0
 * are skipped; errors as for mkp_gemm, before anything is written.
 */
int mkp_gemm_grouped(int64_t groups, int64_t M, int64_t K,
                     const void *A, int64_t lda,
                     const int64_t *N, const void *const *B, const int64_t *ldb,
                     float *const *C, const int64_t *ldc,
                     void *stream);

/* As mkp_gemm_grouped with each B_g given as N_g x K (ldb_g >= K). */
int mkp_gemm_grouped_bt(int64_t groups, int64_t M, int64_t K,
                        const void *A, int64_t lda,
                        const int64_t *N, const void *const *B, const int64_t *ldb,
                        float *const *C, const int64_t *ldc,
                        void *stream);

/* The plan of a grouped call (JSON as mkp_plan_describe; one region spanning
 * the sum of the widths).  flags: MKP_PLAN_B_NK for mkp_gemm_grouped_bt. */
int mkp_plan_describe_grouped(int64_t groups, int64_t M, int64_t K, const int64_t *N, int flags,
                              char *buf, size_t len);

/*
 * Describe the plan the polymerizer picks for a shape, without launching.
 * align_flags: bit0 = A rows 16-byte aligned, bit1 = B rows, bit2 = C rows
 * (pass 7 for aligned operands); MKP_PLAN_B_NK plans for mkp_gemm_bt.
 * Writes NUL-terminated JSON into buf:
 *   {"pattern":..., "cost_us":..., "plan_us":..., "regions":[{"m0","n0","m",
 *    "n","kernel","uM","uN","uK","s","steps","tasks","waves","wave_factor",
 *    "cost_us"}...], "transpose_b": bool [, "transpose_us"], "fused": bool}
 * transpose_b: a K x N B is first copied into N x K workspace rows and the
 * regions run on N x K kernels (the cheaper plan by the cost model).
 * fused: the two regions of a Pattern II plan run in one launch of a
 * two-tile kernel (option "fuse_regions").
 * Uses the active performance table (calibrated, or the built-in analytic
 * one).  Pure host code: needs no GPU.  Returns MKP_OK, MKP_ERR_INVALID_ARG
 * or MKP_ERR_BUFFER.
 */
int mkp_plan_describe(int64_t batch, int64_t M, int64_t N, int64_t K, int align_flags,
                      char *buf, size_t len);

/*
 * As mkp_plan_describe but with a caller-given performance table (text, the
 * format read by mkp_load_calibration) and the pruned or the exhaustive
 * search (flags & MKP_PLAN_EXHAUSTIVE: every candidate is scored, the
 * modelled side of the page's ORACLE variant of section 5 "cost-model
 * effectiveness"); flags & MKP_PLAN_B_NK restricts the search to the
 * table's N x K kernels.  Kernel names in the table need not exist in the
 * library: nothing is launched.  Pure host code.
 */
int mkp_plan_with_table(const char *table_text, int flags,
                        int64_t batch, int64_t M, int64_t N, int64_t K,
                        char *buf, size_t len);

/*
 * Load a performance table (MikPoly page, section 3 "micro-kernel
 * performance model": g_predict per micro-kernel over t K-steps) from a text
 * file; path NULL reloads the table that ships with the library, or the
 * file the environment variable MKP_CALIB names (which must then be
 * readable: only a missing shipped table falls back, silently, to analytic
 * estimates).  Lines:
 *   device <cus>                     launch_us <us>
 *   reduce <launch_us> <GB/s>        splitk <s1> <s2> ...
 *   patterns I II-M II-N             kernel <name> <uM> <uN> <uK> <wg_per_cu> [kn|nk]
 *   g <name> <t>:<us> <t>:<us> ...   measured <TFLOP/s> <GB/s>
 *   tail <name> <f>:<r> ...          tailx <name> <f>:<r> ...
 *   transpose <launch_us> <GB/s>     (copy of a K x N B into N x K)
 *   pair <name a> <name b>           (a and b can share one launch)
 * (kn / nk: the kernel takes B as K x N, the default, or as N x K; tail and
 * tailx: time of a wave filling a fraction f < 1 of the slots, on its own or
 * after full waves, relative to a full wave.)  Kernels named here must exist
 * in the library with the same tile and layout; library kernels the table
 * does not list get analytic estimates.  Each pair
 * must be one the library compiles into a two-tile kernel (same layout and
 * resident workgroups per CU); a table without pair lines gets all of the
 * library's pairs whose kernels it prices with equal workgroups per CU.
 * Clears the plan cache.
 */
int mkp_load_calibration(const char *path);

/*
 * Offline stage: measure g for every library kernel on the current device
 * and write the table to `path` (20 warm-up launches per point, as the page's
 * evaluation does).  Synchronous; uses the null stream.  Returns MKP_OK or an
 * error; the new table becomes active.
 */
int mkp_calibrate(const char *path, int max_points);

/* Set an option: "force_kernel" (kernel name or ""), "force_splitk" (integer,
 * 0 = free), "patterns" ("I" or "I,II"), "exhaustive" (0/1),
 * "splitk_max" (integer), "trace" (0/1, see mkp_trace_dump), "fused_reduce"
 * (0 = split-K partials summed by a second launch, the default; 1 = summed
 * by the last-arriving workgroup of each tile, which on MI355X costs more in
 * L2 write-back than the second launch), "pack_unaligned" (1 = an operand
 * whose rows are not 16-byte aligned, that several tiles re-read and
 * whose K is at least 512 is first copied into aligned workspace rows, the
 * default; 0 = such operands are read element by element).
 * "transpose_b" (0 = K x N calls always run on K x N kernels; 1 = the
 * default: a K x N call may copy B into N x K workspace rows and run on the
 * N x K kernels, when the table prices the copy and the model finds it
 * cheaper; 2 = always, whenever an N x K plan exists).
 * "nt_stores" (how the GEMM kernels and the split-K second pass write C: a
 * sum of bits, 0 = ordinary stores everywhere, kept in the L2 until the
 * kernel's end writes them back; 1 = streaming stores for the final C where
 * its rows are whole 128-byte lines (ldc and the batch stride multiples of
 * 32 floats, the region's first element 128-byte aligned); 2 = for the final
 * C wherever its rows are 16-byte aligned; 4 = for split-K partials; 8 = only
 * in regions of more than one wave of workgroups; 16 = only where the
 * region's C is at most 32 MB; 32 = split-K partials written through to the
 * level every XCD shares, where the second pass reads them; the default is
 * 33).
 * "fuse_regions" (0 = the default: every region of a plan is a launch of its
 * own; 1 = a Pattern II plan over a kernel pair may run both regions in one
 * launch, the second region's workgroups taking the slots the first
 * region's last wave leaves free, when the cost model -- launch + the
 * merged-wave makespan of both regions' tasks + reductions -- finds it
 * cheaper; off by default because on the encoder-linear sweep it measured no
 * faster than two launches).
 * Cost-model evaluation (MikPoly page, section 5 "cost-model effectiveness":
 * the WAVE and PIPE ablations and the ORACLE that measures candidates):
 * "cost_model" ("full" = f_wave * f_pipe, the default; "wave" = f_wave with
 * f_pipe taken as 1 us; "pipe" = f_pipe with f_wave taken as 1; the launch
 * and split-K reduction terms stay in all three; the ablations search the
 * space without pruning), "plan_rank" (0 = the cheapest plan, the default;
 * r > 0 = the r-th cheapest of every candidate of the space, each region
 * with each of its split factors, ties in enumeration order, so that a
 * caller can launch and time candidates one by one; a rank beyond the
 * candidate count makes the GEMM fail with MKP_ERR_UNSUPPORTED).  Both also
 * apply to mkp_plan_with_table, whose JSON then carries "rank" and
 * "candidates".  Every option except "trace", "fused_reduce", "nt_stores"
 * and "pack_unaligned" clears the plan cache.  Returns MKP_OK or
 * MKP_ERR_INVALID_ARG / MKP_ERR_UNSUPPORTED. */
int mkp_set_option(const char *key, const char *value);

/* Number of micro-kernels in the library and the name of kernel i
 * (NULL if out of range).  The string is static. */
int mkp_kernel_count(void);
const char *mkp_kernel_name(int i);

/* Drop every cached plan and free split-K workspaces (synchronises the
 * streams that own them). */
void mkp_cache_clear(void);

/* JSON counters: cache hits/misses, plans built, planning time, launches. */
int mkp_stats(char *buf, size_t len);

/* Launch trace (option "trace" = 1): every kernel launch (micro-kernels,
 * "<a>+<b>" for both regions in one launch of a kernel pair,
 * "splitk_reduce", "zero_fill", "pack_rows", "transpose_b") is bracketed by
 * HIP events on its stream.  Waits for the recorded launches, writes a JSON
 * list [{"kernel","call","us","flops","bytes"}...] ("call": sequence number
 * of the GEMM call that made the launch; algorithmic work per launch:
 * 2*m*n*K flops; 2mK + 2Kn + 4mn bytes) and clears the record. */
int mkp_trace_dump(char *buf, size_t len);

/* Thread-local message of the last error on this thread ("" if none). */
const char *mkp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MKP_H */
