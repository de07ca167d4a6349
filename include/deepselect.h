/*
 * deepselect.h -- C ABI of the MI355X (gfx950) DeepSelect batched row-wise top-k.
 *
 * The operation is DeepSelectTopk of the DeepSelect deep-dive (PFCCLab/DeepSelect,
 * section "算法"): for each row, scan its B-element blocks once in a random order
 * that does not depend on the data, admit the elements greater than a rising
 * threshold T into an on-chip candidate buffer, and whenever the buffer holds
 * k + B2 or more entries shrink it to its k largest with a radix select and set
 * T to the k-th value. The last step selects k once more. The result is exactly
 * the k largest values of the row (the "Top K Selection" problem of
 * "CUDA 算子笔记 4", milkfeng.top).
 *
 * Conventions shared by every entry point
 *   - All pointers named x, out_vals, out_idx, stats and workspace are DEVICE
 *     pointers on the current HIP device. The library never copies them to the
 *     host and never frees them; the caller owns them.
 *   - Row r of the input is x[r*row_stride .. r*row_stride + N) (row_stride in
 *     elements, >= N). Elements are float32 (DS_F32) or bfloat16 (DS_BF16).
 *   - Output row r is out_vals[r*k .. r*k+k) (same element type as x, the exact
 *     bit pattern of the chosen input element) and out_idx[r*k .. r*k+k) (int32
 *     column in [0, N)). The k entries of a row come in no particular order.
 *     When several elements tie at the k-th value any of them may be returned;
 *     the choice is deterministic for a given input, k, B, B2, seed and split.
 *   - Values are ordered by the order-preserving unsigned key of "CUDA 算子笔记 4"
 *     section "改造 Radix Sort" (float_to_key): float order, with -0 < +0, a
 *     positive NaN above +inf and a negative NaN below -inf.
 *   - seed fixes the random block order (a SplitMix64 hash of seed, row and
 *     block id, sorted); the result set does not depend on it, the cost does.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Results are valid after the stream reaches the call; x must not
 *     change before then. Nothing is copied device-to-host.
 *   - Every argument is checked on the host before any HIP call; a rejected call
 *     enqueues nothing. No C++ exception crosses this interface.
 *   - Entry points are thread-safe. The library-owned workspace of split rows
 *     is kept per (device, stream) -- per thread as well for
 *     hipStreamPerThread, whose one handle names a different stream in each
 *     thread -- so calls sharing it are ordered by their stream; it is
 *     allocated (hipMalloc) the first time a shape needs it and grown when a
 *     later shape needs more. A call holds the library's workspace lock from
 *     choosing its workspace until its kernels are queued, and a call that
 *     grows a workspace synchronises that stream before freeing the old one,
 *     so no queued kernel ever uses freed memory.
 *   - A call that needs no workspace (one part per row) or is given a caller
 *     workspace enqueues kernel launches only (no allocation, no memset, no
 *     copy), so it may be captured into a HIP graph and replayed; each replay
 *     recomputes the result from the input as it is at replay time.
 */
#ifndef DEEPSELECT_H
#define DEEPSELECT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DS_F32 = 0, DS_BF16 = 1 } ds_dtype_t;

typedef enum {
    DS_OK = 0,
    DS_ERR_NULL = -1,        /* a required pointer is NULL */
    DS_ERR_DTYPE = -2,       /* dtype not DS_F32 / DS_BF16 */
    DS_ERR_SHAPE = -3,       /* batch < 0, N < 1, N >= 2^31, row_stride < N, misaligned x */
    DS_ERR_K = -4,           /* k < 1 or k > N (the pseudo-code's require line) */
    DS_ERR_BLOCK = -5,       /* B < 1 or B2 < 1, or a forced split the row cannot take */
    DS_ERR_UNSUPPORTED = -6, /* on-chip buffer k+B+B2 (or the block order) exceeds LDS */
    DS_ERR_HIP = -7,         /* a HIP call failed (allocation, attribute, launch) */
    DS_ERR_WORKSPACE = -8,   /* caller workspace smaller than deepselect_workspace_bytes */
    DS_ERR_SCRATCH = -9      /* deepselect_topk_noalloc: the split workspace does not fit the
                                static scratch (deepselect_scratch_bytes), or a workspace was passed */
} ds_status_t;

/* Per-row statistics written when ds_options_t.stats is set: four uint64 per row,
 * in this order (the quantities of the deep-dive's section
 * "RadixSelectTopK 总处理元素数的期望上界"):
 *   W        total input length of every RadixSelectTopK call, the final one included
 *   A        elements admitted into the candidate buffer
 *   R        RadixSelectTopK calls inside the loop (compactions)
 *   MAX_LEN  largest candidate-buffer length reached
 * With split > 1 the row's figures add up its parts and the merge (MAX_LEN: max). */
enum { DS_STAT_W = 0, DS_STAT_A = 1, DS_STAT_R = 2, DS_STAT_MAX_LEN = 3, DS_STATS_PER_ROW = 4 };

typedef struct ds_options {
    /* Parts per row (the deep-dive's "实现" section, last paragraph: a row cut into
     * parts whose top-k are gathered and reduced). 0 = library choice
     * (deepselect_plan_split with the device's compute-unit count). A forced value
     * must satisfy 1 <= split <= ceil(N/B) and leave every part >= k elements,
     * else DS_ERR_BLOCK. */
    int32_t split;
    /* Waves per workgroup of the streaming kernel: 0 = library choice, else 4
     * or 8 (DS_ERR_BLOCK otherwise). Shapes the streaming kernel does not take
     * (rows not 16-byte aligned, N*size or B*size not a multiple of 16, blocks
     * over 8 KiB) run the generic 4-wave kernel whatever is asked. */
    int32_t waves;
    /* Device pointer to batch*4 uint64 (layout above), or NULL for no statistics. */
    uint64_t *stats;
    /* Device workspace for split rows, or NULL for the library-owned one.
     * Size from deepselect_workspace_bytes; no initial contents are needed. It
     * holds every part's results (up to k), their count, the part's k-th and
     * largest keys and statistics between the part kernel and the merge
     * (the merge kernel, or for rows of two bfloat16 parts the part that ends
     * last), and the rows' cells (shared thresholds and the count of a row's
     * ended parts), so it must not be shared by calls that may overlap. */
    void *workspace;
    size_t workspace_bytes;
    /* Kernel: 0 = library choice; 1 = ring streaming (blocks copied HBM -> LDS
     * into a per-wave ring; DS_ERR_UNSUPPORTED when the ring does not fit in
     * LDS); 2 = register streaming (blocks held in registers); 3 = generic
     * (the workgroup shares each block; any layout). 1 and 2 apply to rows the
     * streaming kernels take (see `waves`); others run the generic kernel.
     * Any other value: DS_ERR_BLOCK. */
    int32_t kernel;
    /* Order of each output row: 0 = no particular order; 1 = descending, equal
     * values by ascending column (the worked example of "CUDA 算子笔记 4",
     * section "Top K Selection", lists its result largest first). The results
     * are sorted in LDS before they are written: next_pow2(k) * 8 more bytes of
     * LDS, so a shape near the limit may give DS_ERR_UNSUPPORTED. The result
     * set is the same either way. Any other value: DS_ERR_BLOCK. */
    int32_t sorted;
    /* Device pointer to batch int32 valid lengths, or NULL (every row has N).
     * Row r is then the prefix x[r*row_stride .. r*row_stride + L_r), with
     * L_r = lengths[r] clamped to [0, N]: DeepSelect runs on it exactly as on a
     * row of L_r elements (its ceil(L_r/B) blocks, cut into the call's split;
     * a part may get fewer than k elements or none), and nothing past it takes
     * part (for example a causal sparse-attention row, which covers only the
     * positions before its query: the use of the deep-dive's section
     * "算法设计背景"). When L_r < k the row's first L_r outputs are its
     * elements and the other k - L_r are fillers: index -1 with the bits of
     * negative infinity. Statistics count what the prefix costs. The array is
     * read by the kernels; the library does not check it on the host. */
    const int32_t *lengths;
    /* Fused sampling over each row's results, for the sampling use of the
     * deep-dive's section "算法设计背景" (top-k over vocabulary logits). Needs
     * sorted = 1 (DS_ERR_BLOCK otherwise) and k <= 1024 (DS_ERR_UNSUPPORTED).
     *   probs       device, batch*k floats, or NULL: the softmax of the row's
     *               results at `temperature` (exp((x_j - max)/temperature)
     *               over their sum, in float32), in output order; 0 for
     *               fillers. A row whose largest value is -inf or NaN gets 0;
     *               when it is +inf, the +inf results share the mass equally
     *               and the others get 0 (the softmax's limit).
     *   temperature > 0 (0 is read as 1).
     *   top_p       in (0, 1] (0 is read as 1): the sample is drawn from the
     *               smallest prefix of the sorted results whose probability
     *               reaches top_p (nucleus sampling).
     *   sample_u    device, batch floats in [0, 1), or NULL: the draw of each
     *               row. The sample is the first position of the kept prefix
     *               whose running sum of exponentials exceeds u times the
     *               prefix's sum (inverse CDF in descending order).
     *   sample_idx  device, batch int32, required with sample_u: the sampled
     *               column (-1 for a row with no finite result).
     * Values outside these ranges: DS_ERR_BLOCK. */
    float *probs;
    float temperature;
    float top_p;
    const float *sample_u;
    int32_t *sample_idx;
    /* Split rows: 1 = the parts of a row share their thresholds (0 = off;
     * other values DS_ERR_BLOCK). In the streaming (ring) kernel a part
     * publishes its T (an atomic maximum on the row's cell) at the start of
     * the step after a compaction raised it above what the cell held, one
     * wave per part copies the cell each step, and from two steps later the
     * part filters its blocks with that key when it is above its own T. Its
     * final select first drops the entries at or below such a key. Any
     * part's k-th value is at most the row's, so the result set is the same;
     * the statistics then depend on timing (W = A + k*R still holds per row,
     * W counting the whole buffer at the final stage).
     * The row cells (128 bytes per row: the shared threshold in the first
     * uint64, and in the ninth the count of the row's ended parts, which
     * rows of two bfloat16 parts merged by their last part use) must be zero
     * when the parts start; the merge kernel, or that last part, leaves them
     * zero. The first 1024
     * cells sit at the start of a library-owned workspace or of the noalloc
     * scratch, where no other array overlaps them, so they are cleared only
     * once: by the first such call that is not under graph capture. Cells
     * beyond 1024 rows, every cell of a caller workspace, and the reserved
     * cells of a call made under capture before that are cleared by one
     * small kernel before the parts. After a launch that fails, the next
     * call clears them again. */
    int32_t share_threshold;
} ds_options_t;

/* Check arguments only (pure host code, no HIP call; usable without a GPU).
 * Returns DS_OK or the status deepselect_topk would return before launching. */
int deepselect_validate(int dtype, int64_t batch, int64_t N, int64_t row_stride, int32_t k,
                        int32_t B, int32_t B2);

/* Batched row-wise top-k of x[batch][N] (see the conventions above). */
int deepselect_topk(const void *x, int dtype, int64_t batch, int64_t N, int64_t row_stride,
                    int32_t k, int32_t B, int32_t B2, uint64_t seed, void *out_vals,
                    int32_t *out_idx, void *stream);

/* deepselect_topk with options (forced split, statistics, caller workspace,
 * sorted output, per-row valid lengths, fused sampling, shared thresholds).
 * opt may be NULL (then identical to deepselect_topk). */
int deepselect_topk_ex(const void *x, int dtype, int64_t batch, int64_t N, int64_t row_stride,
                       int32_t k, int32_t B, int32_t B2, uint64_t seed, void *out_vals,
                       int32_t *out_idx, void *stream, const ds_options_t *opt);

/* deepselect_topk_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It calls no hipMalloc, hipFree or other allocating routine. The
 * workspace of split rows (every part's results, counts, k-th and largest
 * keys, statistics and shared-threshold cells) lives in a static device array of
 * 8 MiB, one copy per GPU the library runs on, kept until the process ends;
 * its device address is looked up once per device on the first call there.
 * Its first 128 KiB hold 1024 reserved row cells (see share_threshold);
 * deepselect_scratch_bytes() is the rest. Arguments and results are those of
 * deepselect_topk_ex with the same options, except:
 *   - opt->workspace must be NULL (else DS_ERR_SCRATCH);
 *   - a call whose split needs more workspace than the scratch holds
 *     (deepselect_workspace_bytes > deepselect_scratch_bytes) returns
 *     DS_ERR_SCRATCH with nothing enqueued; force a smaller opt->split or use
 *     deepselect_topk_ex.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents. A call needs none of them except the reserved cells, which
 * every call leaves zero (share_threshold says when they are cleared). Calls
 * that may overlap on one GPU (other streams, other threads) race on it:
 * order them.
 * Calls with one part per row use no scratch. */
int deepselect_topk_noalloc(const void *x, int dtype, int64_t batch, int64_t N, int64_t row_stride,
                            int32_t k, int32_t B, int32_t B2, uint64_t seed, void *out_vals,
                            int32_t *out_idx, void *stream, const ds_options_t *opt);

/* Bytes of the static scratch deepselect_topk_noalloc has for the workspace
 * of a call on each GPU (8 MiB less its 128 KiB of reserved cells): a call fits
 * when deepselect_workspace_bytes for its shape is at most this. */
size_t deepselect_scratch_bytes(void);

/* The split factor the library picks for this shape on a device with num_cus
 * compute units (pure host code). Returns >= 1, or a negative status. */
int deepselect_plan_split(int dtype, int64_t batch, int64_t N, int32_t k, int32_t B, int32_t B2,
                          int32_t num_cus);

/* Workspace bytes a call with this shape and split needs (0 when split == 1).
 * Pure host code. Returns 0 for invalid arguments as well. */
size_t deepselect_workspace_bytes(int dtype, int64_t batch, int64_t N, int32_t k, int32_t B,
                                  int32_t B2, int32_t split);

/* Dynamic LDS bytes one workgroup of this shape uses (pure host code; 0 if invalid). */
size_t deepselect_lds_bytes(int dtype, int64_t N, int32_t k, int32_t B, int32_t B2,
                            int32_t split);

/* Static description of a status code (never NULL). */
const char *deepselect_status_string(int status);

/* Free every library-owned workspace (all devices and streams). Must not be
 * called while a call using one is still queued. */
void deepselect_release(void);

#ifdef __cplusplus
}
#endif

#endif /* DEEPSELECT_H */
