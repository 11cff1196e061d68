/*
 * online_softmax.h -- C ABI of the MI355X (gfx950) row-wise softmax library
 * built on the online normalizer.
 *
 * The method (each entry point below cites the passage it implements):
 *   - "OnlineSoftmax: Online normalizer calculation for softmax" (paper
 *     summary), section 3.1: one pass folds a row into (m, d), m the running
 *     maximum and d = sum_j e^{x_j - m}, by
 *         m_j = max(m_{j-1}, x_j),  d_j = d_{j-1} e^{m_{j-1} - m_j} + e^{x_j - m_j};
 *     section 3.3: partial states merge with the associative, commutative
 *         (m1,d1) (+) (m2,d2) = (max, d1 e^{m1-max} + d2 e^{m2-max});
 *     a second pass writes y_i = e^{x_i - m} / d.
 *   - "第 7 课：Online Softmax 与可结合状态", section 3: the identity state
 *     is (-inf, 0).
 *   - The paper summary, section 4 "Softmax and top-k fusion": one pass keeps
 *     the K largest logits next to (m, d); only K probabilities are written.
 *   - The paper summary, section 2, and "5.2 Hiện thực và tối ưu CUDA Online
 *     Softmax", section 1.1: safe softmax in three passes (max, sum, divide),
 *     the baseline.
 *   - "6.2 FlashAttention V2 chi tiết", sections 6.1 and 7.1: the per-row
 *     logsumexp L = m + log(d) kept in place of m and d.
 *
 * Conventions shared by every entry point
 *   Layout     row-major, contiguous, row stride == cols elements.
 *   Pointers   device pointers (HIP device memory of the current device) unless
 *              stated; the caller allocates and owns every buffer.  The library
 *              allocates no device memory.
 *   Stream     `stream` is a hipStream_t passed as void* (NULL = null stream).
 *              Calls are asynchronous on that stream and never synchronise;
 *              results are valid once the stream reaches the call.
 *   dtype      OS_F32: float in, float out.  OS_BF16: bfloat16 in and out
 *              (raw 16-bit patterns), fp32 arithmetic inside, output rounded to
 *              nearest-even.
 *   Aliasing   `in == out` (exact alias) is allowed for every forward entry
 *              point (plain, tuned, logsumexp, split) and the safe baseline;
 *              any other overlap is undefined.
 *   Sizes      0 <= cols <= OS_MAX_COLS; rows * cols * element size must fit in
 *              int64.
 *   Empty      rows == 0, or cols == 0 for the forward/safe entry points, is a
 *              no-op returning OS_OK (pointers may then be NULL).
 *   Special    a row containing NaN or +inf gives NaN for the whole row; -inf
 *   values     entries get probability 0; a row with no entry above -inf has
 *              state (-inf, 0) and softmax NaN (0/0).
 *   Errors     a negative status; nothing is launched on an error found while
 *              checking arguments, which happens before any HIP call.
 *              os_last_error() describes the last failure on the calling thread.
 *   Alignment  pointers must be aligned to their element size.  Every row is
 *              moved with 128-bit accesses: rows whose starts are not 16-byte
 *              aligned are read as the 16-byte blocks they overlap, and a
 *              kernel that gives a whole workgroup to one row may start at
 *              the 128-byte line holding the row's first element.  So a read
 *              may touch up to 127 bytes before a row range's first element
 *              (within that element's 128-byte line) and up to 15 bytes after
 *              its last (within its 16-byte block), and so never leaves a
 *              mapped page.  Writes touch only output elements:
 *              whole blocks where out has in's offset within its 16-byte
 *              block, single elements at the ends of rows and when the offsets
 *              differ.  Several short rows handled together are written as
 *              whole blocks of their common run, with single elements only at
 *              the run's two ends.
 */
#ifndef ONLINE_SOFTMAX_H
#define ONLINE_SOFTMAX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define OS_OK 0
#define OS_EINVAL (-1)       /* bad argument (null pointer, size, dtype, K, misalignment) */
#define OS_EUNSUPPORTED (-2) /* a requested kernel shape is not built into the library */
#define OS_ELAUNCH (-3)      /* the HIP runtime rejected a launch or a device query */

/* element types */
#define OS_F32 0
#define OS_BF16 1

/* largest K accepted by os_softmax_topk */
#define OS_TOPK_KMAX 32

/* most workgroups one row may be split over in os_softmax_topk_split */
#define OS_TOPK_MAX_SPLITS 16
/* most workgroups one row may be split over in os_softmax_forward_split */
#define OS_FWD_MAX_SPLITS 256

/* largest row length (columns) accepted by every entry point: 2^28 */
#define OS_MAX_COLS (1LL << 28)

/*
 * y = softmax(x) row by row with the online normalizer (paper summary,
 * sections 3.1 and 3.3; the normalising pass as in "5.2 Hiện thực và tối ưu
 * CUDA Online Softmax", section 2.2).
 *   in, out   [rows, cols] of `dtype`.
 *   The kernel is chosen from `cols`, `dtype` and the row alignment: rows of
 *   up to 32768 fp32 or 65536 bf16 elements stay in registers and are read
 *   from HBM once (several rows per wavefront, one wavefront per row, or one
 *   workgroup per row); rows of up to 262144 elements keep a leading part in
 *   registers (32768 to 65536 fp32 elements by row length, 57344 bf16) and
 *   the next 32768 fp32 or 65536 bf16 in LDS, and read the rest twice (fp32
 *   rows of up to 65536 and bf16 rows of up to 122880 are so read once);
 *   longer rows are streamed in two passes (fold, then normalise), reading
 *   the row twice.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_softmax_forward(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                       void *stream);

/*
 * Same computation as os_softmax_forward with an explicit kernel shape, for
 * tests and tuning.
 *   lanes_per_row   lanes that share one row: 4, 8, 16, 32, 64, 128, 256, 512
 *                   or 1024 (register-resident kernels), or 0 for the
 *                   streaming two-pass kernel.
 *   vecs_per_lane   16-byte vectors held per lane (1, 2, 4, 8 or 16, 5 on 256
 *                   lanes, 5 or 6 on 512 and 1024 lanes; only the combinations
 *                   built into the library are accepted).  The
 *                   shape must hold the row: lanes_per_row * vecs_per_lane *
 *                   VEC >= cols, VEC = 16 / element size, and >= cols + VEC - 1
 *                   when the row starts are not all 16-byte aligned (such a
 *                   row may span one more 16-byte block).  Ignored when
 *                   lanes_per_row == 0.
 *   grid_blocks     workgroups to launch (grid-stride over rows); 0 = automatic.
 *   Returns OS_OK, OS_EINVAL (shape too small or grid_blocks < 0),
 *   OS_EUNSUPPORTED (shape not built), or OS_ELAUNCH.
 */
int os_softmax_forward_tuned(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                             int lanes_per_row, int vecs_per_lane, int grid_blocks, void *stream);

/*
 * The shape os_softmax_forward uses for rows of `cols` elements of `dtype` in
 * an array whose base is 16-byte aligned (the shape depends on whether the row
 * starts are all 16-byte aligned, i.e. on cols * element size % 16 here).
 * Short rows that are not aligned may get a shape that holds only `cols`
 * elements per row, not the extra block they span: those are read through
 * LDS.  Host only: no HIP call.
 *   *lanes_per_row, *vecs_per_lane receive the shape (0, 0 for rows longer
 *   than the register-resident kernels hold).
 *   Returns OS_OK or OS_EINVAL.
 */
int os_forward_plan(int64_t cols, int dtype, int *lanes_per_row, int *vecs_per_lane);

/*
 * Per-row normaliser state (m, d) from the fold and the (+) merge alone, no
 * output pass (paper summary, sections 3.1-3.3).
 *   in      [rows, cols] of `dtype`.
 *   m, d    [rows] float each.  A row with no entry above -inf (or cols == 0)
 *           gets the identity (-inf, 0).  A row holding NaN or +inf gets d NaN;
 *           its m is the largest entry other than NaN, or -inf if there is
 *           none above -inf (so also when that entry is -FLT_MAX and the row
 *           holds a NaN).
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_softmax_stats(const void *in, float *m, float *d, int64_t rows, int64_t cols, int dtype,
                     void *stream);

/*
 * Forward with the per-row logsumexp L = m + ln d = ln(sum_j e^{x_j}), the
 * statistic "6.2 FlashAttention V2 chi tiết" keeps in place of m and d for
 * the backward pass (sections 6.1 and 7.1), written by the same launch as y.
 *   in      [rows, cols] of `dtype`.
 *   out     [rows, cols] of `dtype`, y as os_softmax_forward writes it, or
 *           NULL to compute L alone (a logsumexp reduction).  in == out is
 *           allowed.
 *   lse     [rows] float, owned by the caller.  -inf for a row with no entry
 *           above -inf (or cols == 0); NaN for a row holding NaN or +inf.
 *           fp32: m + log2(d) * ln 2 rounded once (fused multiply-add).
 *   Returns OS_OK, OS_EINVAL (lse NULL or misaligned, or as for the
 *   forward), or OS_ELAUNCH.
 */
int os_softmax_forward_lse(const void *in, void *out, float *lse, int64_t rows, int64_t cols, int dtype,
                           void *stream);

/*
 * The forward with each row split over `splits` workgroups, for batches with
 * too few rows to occupy the GPU (the paper summary, section 3.3: (+) lets any
 * partition of a row be folded separately and merged; "5.2 Hiện thực và tối ưu
 * CUDA Online Softmax", section 7.1, on several blocks per row).  Two launches
 * on `stream`: each slice folds its (m, d) into the workspace, then each slice
 * merges its row's states in a fixed order and writes its part of y.  The
 * input is read twice and y written once.
 *   in, out, rows, cols, dtype   as os_softmax_forward (in == out allowed).
 *   splits      1..OS_FWD_MAX_SPLITS (1 = os_softmax_forward; workspace unused).
 *   workspace   device memory of at least
 *               os_softmax_forward_workspace_bytes(rows, splits) bytes, 8-byte
 *               aligned, owned by the caller; no initialisation needed.  It is
 *               in use until the second launch completes: calls that overlap
 *               on other streams need workspaces of their own.
 *   Returns OS_OK, OS_EINVAL (bad splits, missing, misaligned or short
 *   workspace, or as for the forward), or OS_ELAUNCH.
 */
int os_softmax_forward_split(const void *in, void *out, int64_t rows, int64_t cols, int dtype, int splits,
                             void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of the device-resident scratch array os_softmax_forward_split_noalloc
 * uses on each GPU (1 MiB): rows * splits * 8 must not exceed it. */
#define OS_STATIC_SCRATCH_BYTES (1LL << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as os_softmax_forward_split, with the slice states kept in a
 * fixed array inside the library instead of a caller's workspace.  The call
 * allocates nothing and calls no allocating routine; each GPU the library
 * runs on holds its own OS_STATIC_SCRATCH_BYTES array until the process ends
 * (its address is looked up on the first call on that device).
 *   in, out, rows, cols, dtype, splits, stream   as os_softmax_forward_split.
 *   The array needs no initialisation (the first launch writes every slice
 *   state before the second reads any) and keeps the last call's contents.
 *   Every call on one GPU shares that GPU's array: calls on one stream are
 *   ordered, but calls that overlap in time on one GPU (different streams)
 *   race and give wrong results.
 *   Returns OS_OK, OS_EINVAL (as os_softmax_forward_split, or
 *   rows * splits * 8 > OS_STATIC_SCRATCH_BYTES), or OS_ELAUNCH.
 */
int os_softmax_forward_split_noalloc(const void *in, void *out, int64_t rows, int64_t cols, int dtype, int splits,
                                     void *stream);

/* Workspace bytes os_softmax_forward_split needs (0 for splits == 1), or
 * OS_EINVAL for rows < 0 or splits outside 1..OS_FWD_MAX_SPLITS.  Host only. */
int64_t os_softmax_forward_workspace_bytes(int64_t rows, int splits);

/* Suggested `splits` for a forward batch (1 = no split).  Host only. */
int os_forward_split_plan(int64_t rows, int64_t cols, int dtype);

/*
 * Fused softmax + top-K in one read of the input (paper summary, section 4):
 * the K largest logits of each row and their probabilities over the WHOLE row,
 * v = e^{u - m} / d (not renormalised over the K).  The full softmax is never
 * written.
 *   in      [rows, cols] float.
 *   probs   [rows, K] float, best first.
 *   idx     [rows, K] int32 column indices, best first.  Order: larger logit
 *           first; equal logits (including -0.0 == +0.0) by lower index first.
 *   K       1 <= K <= min(cols, OS_TOPK_KMAX).
 *   Rows containing NaN give NaN probabilities; their indices are K distinct
 *   columns of the row, which ones unspecified.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_softmax_topk(const float *in, float *probs, int32_t *idx, int64_t rows, int64_t cols, int K,
                    void *stream);

/*
 * os_softmax_topk with each row split over `splits` workgroups, for batches
 * too small to occupy the GPU with one workgroup per row (the pages' "several
 * blocks per row": "5.2 Hiện thực và tối ưu CUDA Online Softmax", section
 * 7.1).  Each workgroup folds a contiguous slice of the row into a state
 * (m, d) and a sorted candidate list and writes both to `workspace`; a
 * second launch on the same stream merges, per row, the slice states with
 * (+) (paper summary, section 3.3) and the lists, in slice order, so results
 * are identical to os_softmax_topk's.
 *   splits      1..OS_TOPK_MAX_SPLITS (1 = os_softmax_topk; workspace unused).
 *   workspace   device memory of at least os_softmax_topk_workspace_bytes()
 *               bytes, 256-byte aligned, owned by the caller; no
 *               initialisation needed.  Calls that may overlap in time
 *               (different streams) need separate workspaces.
 *   Other arguments, results and errors as os_softmax_topk; a missing or
 *   short workspace is OS_EINVAL.
 */
int os_softmax_topk_split(const float *in, float *probs, int32_t *idx, int64_t rows, int64_t cols, int K,
                          int splits, void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of workspace os_softmax_topk_split needs (0 for splits == 1), or
 * OS_EINVAL for bad arguments.  Host only. */
int64_t os_softmax_topk_workspace_bytes(int64_t rows, int K, int splits);

/* Suggested `splits` for a top-K batch (1 = no split).  Host only. */
int os_topk_plan(int64_t rows, int64_t cols, int K);

/*
 * The fused softmax + top-K for fp32 or bf16 logits (the paper summary,
 * section 4), with an optional split as in os_softmax_topk_split.  bf16
 * inputs widen exactly to fp32; the arithmetic, the ranking (value desc,
 * index asc; bf16 rows tie far more often) and the outputs are those of
 * os_softmax_topk.
 *   in      [rows, cols] of `dtype`, aligned to its element size.
 *   dtype   OS_F32 or OS_BF16.
 *   probs, idx, rows, cols, K, splits, workspace, workspace_bytes, stream
 *           as os_softmax_topk_split (the workspace does not depend on dtype).
 *   Returns OS_OK, OS_EINVAL (as os_softmax_topk_split, or an unknown dtype),
 *   or OS_ELAUNCH.
 */
int os_softmax_topk_ex(const void *in, int dtype, float *probs, int32_t *idx, int64_t rows, int64_t cols, int K,
                       int splits, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Baseline: safe softmax in three passes over the input in global memory
 * (maximum, sum of e^{x-m}, normalise and store), as in the paper summary,
 * section 2, and "5.2 Hiện thực và tối ưu CUDA Online Softmax", section 1.1.
 * It reads every row three times (re-reads of short rows may hit in cache),
 * with the same lanes-per-row geometry os_softmax_forward picks; same
 * arguments and results as os_softmax_forward.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int safe_softmax_forward(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                         void *stream);

/*
 * Baseline: the unshifted ("original") softmax y_i = e^{x_i} / sum_j e^{x_j}
 * of the paper summary, section 2, in two passes over the input in global
 * memory (the sum of e^x, then normalise and store) with no maximum
 * subtracted: the third algorithm of the paper summary's section 5
 * comparison.  Same arguments, layout and geometry as safe_softmax_forward.
 *   Results match the safe and online forms only where e^x is finite and
 *   normal in fp32 (about -87 < x < 88.7 for every entry); past that, e^x
 *   overflows to +inf or underflows to 0 and rows turn to NaN or lose
 *   accuracy, the failure the page describes.  Not for production use.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int naive_softmax_forward(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                          void *stream);

/*
 * Top-K selection alone: the K largest entries of each row under (value desc,
 * index asc), written as the entries themselves with their columns; no
 * exponential and no normaliser.  This is the TopK stage of the unfused
 * pipelines in the paper summary's section 4 access table (softmax written
 * out, then TopK reading the probabilities), the comparison point of the
 * fused os_softmax_topk.  One read of the input; the fused kernel's filter,
 * lists and merge with the fold switched off.
 *   in      [rows, cols] of `dtype` (OS_F32 or OS_BF16, widened exactly).
 *   vals    [rows, K] float, best first: the selected entries.
 *   idx     [rows, K] int32 columns, best first; equal entries (including
 *           -0.0 == +0.0) by lower column first.
 *   K       1 <= K <= min(cols, OS_TOPK_KMAX).
 *   Rows containing NaN give K distinct in-row columns, which ones and their
 *   values unspecified.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_topk_select(const void *in, int dtype, float *vals, int32_t *idx, int64_t rows, int64_t cols, int K,
                   void *stream);

/*
 * Plain device copy of `bytes` bytes with 128-bit accesses: the reference
 * read+write kernel used to calibrate traffic counters and as a bandwidth
 * ceiling.  src and dst must be 16-byte aligned, bytes a multiple of 16,
 * no overlap.  Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_device_copy(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * Plain device read of `bytes` bytes with 128-bit accesses (4 KiB tiles,
 * 256-thread workgroups striding over them, at most 2048 workgroups): the
 * read-only bandwidth reference for kernels that only read, such as the fused
 * top-K.  src 16-byte aligned, bytes a multiple of 16.
 *   sink         device floats receiving one sum per wave (values carry no
 *                meaning; they keep the loads from being dropped).
 *   sink_floats  capacity of sink: at least 4 * min(2048, ceil(bytes / 4096)).
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_device_read(const void *src, int64_t bytes, float *sink, int64_t sink_floats, void *stream);

/*
 * Device copy of `rows` rows of `row_bytes` bytes each with the access pattern
 * of the register-resident forward on rows up to 128 KiB: one 1024-lane
 * workgroup per row, eight 16-byte vectors per lane, every load of a row
 * issued before any of its stores.  A bandwidth reference: the ceiling of that
 * pattern, next to os_device_copy's (4 KiB tiles, one vector per lane).
 * row_bytes a multiple of 16 and at most 131072; src and dst 16-byte aligned,
 * no overlap.  Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_device_copy_rows(const void *src, void *dst, int64_t rows, int64_t row_bytes, void *stream);

/* longest query or key sequence accepted by os_attention_forward: 2^22 */
#define OS_ATTN_MAX_SEQ (1LL << 22)

/*
 * Attention forward with the online normalizer: per head,
 *     O = softmax(scale * Q K^T) V,   L = m + ln l  (the row's logsumexp),
 * the self-attention of the paper summary's section 7.1, computed without
 * forming Q K^T in memory by the tiled (m, l, o~) recurrence of its section
 * 7.2.3 in the delayed-rescaling form of "6.2 FlashAttention V2 chi tiết"
 * (sections 3.2 and 6.1: the running output is rescaled by e^{m_old - m_new}
 * per key tile and divided by l once at the end; the logsumexp is the
 * statistic of its section 7.1).  The two products run on the bf16 matrix
 * cores with fp32 accumulation; the softmax state is fp32.
 *   q        [heads, nq, head_dim] bf16 (raw 16-bit patterns).
 *   k, v     [heads, nk, head_dim] bf16.
 *   o        [heads, nq, head_dim] bf16, written (rounded to nearest-even).
 *            o may be q itself; no other overlap.
 *   lse      [heads, nq] float, or NULL: L = scale * max_j (q.k_j) + ln l.
 *   head_dim 128 (the only one built).
 *   scale    > 0 and finite (1/sqrt(head_dim) on the pages).
 *   causal   non-zero: key j is hidden from query row i when j > i ("6.2
 *            FlashAttention V2 chi tiết", section 5; key tiles wholly above
 *            the diagonal are skipped); needs nq == nk.
 *   heads == 0 or nq == 0 is a no-op; otherwise 1 <= nk, and nq, nk <=
 *   OS_ATTN_MAX_SEQ.  q, k, v, o 16-byte aligned.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_attention_forward(const void *q, const void *k, const void *v, void *o, float *lse, int64_t heads,
                         int64_t nq, int64_t nk, int head_dim, float scale, int causal, void *stream);

/*
 * Microbenchmark of the hardware exponential (v_exp_f32), the arithmetic
 * ceiling beside HBM bandwidth: every element of a fold costs one (the paper
 * summary's section 3 counts the recurrence's extra work per element; "5.2
 * Hiện thực và tối ưu CUDA Online Softmax", section 4.4, weighs the extra
 * exponentials against the bytes saved).  `workgroups` 256-thread workgroups;
 * every lane runs `iters` rounds of one exponential and one fused
 * multiply-add on each of `chains` values (1: one dependent chain, latency;
 * 8: independent chains, throughput), so a launch performs
 * workgroups * 256 * iters * chains exponentials.
 *   out         [workgroups * 256] float, one result per lane (kept so that
 *               no work is dropped; its values carry no meaning).
 *   workgroups  1..2^20;  iters >= 1;  chains 1 or 8.
 *   Returns OS_OK, OS_EINVAL, or OS_ELAUNCH.
 */
int os_bench_exp(float *out, int64_t workgroups, int iters, int chains, void *stream);

/* Message for the last failing call on this thread ("" if none).  The pointer
 * stays valid until the next call on the same thread. */
const char *os_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int os_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ONLINE_SOFTMAX_H */
