/*
 * pa.h - C ABI of the MI355X (gfx950) paged decode attention library (libpa.so).
 *
 * Sources for what is computed (web pages describing the samir-vllm teaching
 * engine; cited by title and section):
 *   [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
 *            Inference - Start here" (memedata.com copy of the project README),
 *            feature list: the KV page pool item, the batched decode item and
 *            the paged decode attention item.
 *   [ARCH]   "samir-vllm: Build LLM Inference From Scratch in C++ and CUDA"
 *            (wpnews.pro), section "Architecture walkthrough", KV cache
 *            paragraph.
 *   [NF]     news-factory.app article on the free LLM-inference course,
 *            section "How does the engine manage KV cache memory?".
 *
 * Data model ([README] KV page pool item; [ARCH]):
 *   - One shared BF16 pool of physical pages.  A page holds 16 tokens of K and
 *     V of one layer.  The K plane and the V plane are two arrays indexed by
 *     the same page id, each laid out as bf16 [num_pages][16][Hkv][D]: a token
 *     row of one page is Hkv*D contiguous values, one KV head's row is D
 *     contiguous values (128 bytes for D = 64).
 *   - A block table per (sequence, layer): int32 [B][max_blocks] for one layer,
 *     entry j is the page of logical tokens 16j .. 16j+15.  Entries at index
 *     >= ceil(L/16) are never read (they may hold -1).  The entries below it
 *     must be page ids in [0, num_pages) and L must be at most 16 * max_blocks:
 *     pa_append, pa_decode, pa_append_decode and pa_rope_append_decode use
 *     them as given, without a device-side check, so a value outside them
 *     reads or writes outside the pools.  pa_fill and pa_rope_append check
 *     both and skip the rows that fail.
 *   - seq_lens: int32 [B], the length of each sequence AFTER this step's
 *     append.  One array serves every layer of a step.
 *   - BF16 values are passed as uint16_t bit patterns.
 *
 * Supported model dimensions: Hkv = 8, D = 64, Hq = 32 (4 query heads per KV
 * head).  The pages fix the model (Llama 3.2 1B, 2048-wide hidden state, 16
 * layers, 2048-token context) but do not print the head counts; 32 x 64 = 2048
 * is the reading used.  Other values return PA_ERR_UNSUPPORTED.
 *
 * Conventions shared by every call:
 *   - Pointers named *_pool, q, k_new, v_new, block_table, seq_lens, out,
 *     part_* and workspace are DEVICE pointers owned by the caller.  The
 *     library allocates, frees and synchronises nothing and keeps no state
 *     between calls beyond a per-device flag (atomic) that the decode
 *     kernels' dynamic LDS limit has been raised and, for
 *     pa_append_decode_noalloc only, its per-device scratch array and that
 *     array's device address; it is reentrant (pa_append_decode_noalloc
 *     calls that overlap on one GPU excepted).
 *   - Arguments are validated on the host before anything is launched; on a
 *     failed check the call returns a negative status and launches nothing.
 *     B == 0 is a valid empty batch: the call returns PA_OK and launches
 *     nothing.  Every array pointer must be 16-byte aligned.
 *   - Work is enqueued on `stream` and runs asynchronously; a launch failure
 *     reported by the runtime returns PA_ERR_LAUNCH.
 *   - Device-side preconditions (the caller's contract, not checked):
 *     0 <= seq_lens[b] <= 16*max_blocks; every block table entry below
 *     ceil(L/16) lies in [0, num_pages); no two (sequence, layer) pairs own the
 *     same page.  Slots the call does not reference may hold anything,
 *     including NaN: they never influence a result.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_PAGE_TOKENS 16
#define PA_HEAD_DIM 64
#define PA_KV_HEADS 8
#define PA_Q_HEADS 32
#define PA_MAX_BLOCKS_LIMIT 4096
#define PA_MAX_DECODE_BATCH 4096
#define PA_MAX_FILL_BATCH 4096
#define PA_MAX_PREFILL_BATCH 4096
#define PA_MAX_PREFILL_ROWS (1 << 30)
#define PA_PREFILL_WEIGHTS_BF16X2 0
#define PA_PREFILL_WEIGHTS_FP16 1
/* Size of the device scratch array behind pa_append_decode_noalloc (64 MiB per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  PA_ERR_UNSUPPORTED = -3, /* dims other than Hq=32, Hkv=8, D=64 */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = -5,      /* the HIP runtime rejected a launch */
  PA_ERR_ALIGN = -6,       /* an array pointer is not 16-byte aligned */
  PA_ERR_REJECTED = -7,    /* pa_sched: the request's budget exceeds the whole pool */
  PA_ERR_BUDGET = -8,      /* pa_sched: growth beyond the request's reserved prefix */
  PA_ERR_STATE = -9,       /* pa_sched: the request is not active */
  PA_ERR_SCRATCH = -10     /* pa_append_decode_noalloc: the call needs more than the fixed scratch */
};

/* Human-readable name of a status code (static string). */
const char* pa_status_string(int status);

/*
 * pa_append - write this step's token of every sequence into its page slot.
 * ([README] KV page pool item: decode appends one new token at its absolute
 * position; [ARCH] KV cache paragraph.)
 *
 * For each b with L = seq_lens[b] >= 1: page = block_table[b][(L-1)/16],
 * slot = (L-1) % 16; k_pool[page][slot][:][:] = k_new[b][:][:] and likewise
 * v_pool from v_new, as a bit copy.  Sequences with L == 0 are skipped.
 *
 *   k_new, v_new  bf16 [B][Hkv][D]
 *   k_pool, v_pool bf16 [num_pages][16][Hkv][D] (written)
 *   block_table   int32 [B][max_blocks] of one layer
 *   seq_lens      int32 [B]
 * The caller assigns the page of block (L-1)/16 before the call whenever
 * (L-1) % 16 == 0 (pages are assigned lazily by the host).
 */
int pa_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
              const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t B,
              int32_t Hkv, int32_t D, int64_t num_pages, hipStream_t stream);

/*
 * pa_rope_append - rotate this step's query and new key by RoPE at the token's
 * absolute position, then write the new K and V into the page slot.
 * ([README] feature list: RoPE is applied to the projected queries and keys
 * before attention; KV page pool item: decode appends one new token at its
 * absolute RoPE position.  The pages print no RoPE constants or pairing.)
 *
 * For each b with L = seq_lens[b] >= 1, pos = L - 1 < max_pos, and a table
 * entry page = block_table[b][pos/16] in [0, num_pages):
 *   q_out[b][h]          = rot(q[b][h])       for the Hq query heads
 *   k_pool[page][slot][g] = rot(k_new[b][g])  slot = pos % 16, g < Hkv
 *   v_pool[page][slot][g] = v_new[b][g]       (bit copy)
 * with, for i < 32, c_i = cos_sin[pos][i] and s_i = cos_sin[pos][32 + i]:
 *   rot(x)[i]      = x[i] c_i - x[i + 32] s_i
 *   rot(x)[i + 32] = x[i + 32] c_i + x[i] s_i
 * Each product and the difference or sum is one FP32 operation rounded to
 * nearest (no fused multiply-add); the result is rounded to BF16 to nearest,
 * ties to even (a NaN stays a quiet NaN).  The table carries the base and any
 * frequency scaling.  Other sequences are skipped: their q_out rows are not
 * written and nothing is appended.
 *
 *   q, q_out      bf16 [B][Hq][D] (q_out written).  q_out may be q itself (the
 *                 rotation is done in place: every row is read before it is
 *                 written) or a buffer disjoint from it; a partial overlap is
 *                 not allowed.
 *   k_new, v_new  bf16 [B][Hkv][D]
 *   cos_sin       fp32 [max_pos][D]
 *   k_pool, v_pool bf16 [num_pages][16][Hkv][D] (written)
 *   block_table   int32 [B][max_blocks] of one layer
 *   seq_lens      int32 [B]
 * B in 0 .. PA_MAX_DECODE_BATCH.  The caller assigns the page of block
 * (L-1)/16 before the call, as for pa_append.  Returns PA_OK, PA_ERR_SHAPE,
 * PA_ERR_UNSUPPORTED, PA_ERR_NULL, PA_ERR_ALIGN or PA_ERR_LAUNCH; nothing is
 * launched for B == 0.
 */
int pa_rope_append(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const float* cos_sin,
                   int32_t max_pos, uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool,
                   const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                   int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, hipStream_t stream);

/*
 * pa_rope_append_decode - pa_rope_append and pa_decode in one launch: q and
 * the new key are rotated by RoPE at position L-1 exactly as pa_rope_append
 * rotates them, the rotated key and the value are appended, and the attention
 * runs with the rotated query.  The pools and out are bit-identical to
 * pa_rope_append followed by pa_decode on its q_out (the rotated q itself is
 * not stored).  ([README] feature list and KV page pool item, as for
 * pa_rope_append; [README] paged decode attention item, as for pa_decode.)
 *
 * Arguments as pa_append_decode, plus cos_sin fp32 [max_pos][D] as for
 * pa_rope_append, with max_pos >= 16 * max_blocks so that the table covers
 * every position the block table can address (else PA_ERR_SHAPE).  Unlike
 * pa_rope_append it skips nothing: every sequence is decoded as pa_decode
 * decodes it.
 */
int pa_rope_append_decode(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
                          const uint16_t* q, const float* cos_sin, int32_t max_pos, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* seq_lens, float scale, float* out, int32_t B,
                          int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, int32_t partition_tokens,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_fill - write a run of consecutive tokens of every sequence into its pages
 * (prefill).  ([README] KV page pool item: prefill fills prompt pages, through
 * the same per-(sequence, layer) block table that decode reads.)
 *
 * Sequence b's run is rows cu_tokens[b] .. cu_tokens[b+1]-1 of k_src / v_src;
 * row i of it is the token at position p = start[b] + i and is bit-copied to
 * k_pool[block_table[b][p/16]][p%16] (likewise V).  The pages' prefill is
 * start = 0 (the whole prompt); a one-token run at position L-1 is pa_append.
 *
 *   k_src, v_src  bf16 [T][Hkv][D], the runs one after another
 *   k_pool, v_pool bf16 [num_pages][16][Hkv][D] (written)
 *   block_table   int32 [B][max_blocks] of one layer
 *   start         int32 [B], or NULL for all 0
 *   cu_tokens     int32 [B+1]: cu_tokens[0] = 0, nondecreasing, cu_tokens[B] = T
 *   B             0 .. PA_MAX_FILL_BATCH; T total rows (0 .. 2^31-17)
 * The caller assigns every page the runs reach before the call.  Rows whose
 * position is negative or past the table, or whose table entry is outside
 * [0, num_pages), are not written.  Runs must not overlap in the pool.
 * Returns PA_OK, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_NULL, PA_ERR_ALIGN
 * or PA_ERR_LAUNCH; nothing is launched for B == 0 or T == 0.
 */
int pa_fill(const uint16_t* k_src, const uint16_t* v_src, uint16_t* k_pool, uint16_t* v_pool,
            const int32_t* block_table, int32_t max_blocks, const int32_t* start, const int32_t* cu_tokens,
            int32_t B, int64_t T, int32_t Hkv, int32_t D, int64_t num_pages, hipStream_t stream);

/*
 * pa_prefill - dense causal attention of whole prompts over their own K and V,
 * with grouped-query heads (prefill).  ([README] feature list: dense causal
 * prefill, grouped-query attention in all layers; Llama 3.2 1B shapes, Hq = 32
 * query heads sharing Hkv = 8 KV heads, D = 64.)
 *
 * Prompt b is rows cu_tokens[b] .. cu_tokens[b+1]-1; row i of it attends rows
 * cu_tokens[b] .. i of the same prompt (the prompt's own positions up to i):
 *
 *   out[i][h][:] = sum_{j = cu_tokens[b]}^{i} softmax_j(scale * q[i][h] . k[j][g]) v[j][g],
 *   g = h / (Hq / Hkv).
 *
 *   q            bf16 [T][Hq][D] (already position-encoded)
 *   k, v         bf16 [T][Hkv][D], the prompts' own keys and values
 *   cu_tokens    int32 [B+1] on the device: cu_tokens[0] = 0, nondecreasing,
 *                cu_tokens[B] = T; empty prompts are allowed
 *   out          fp32 [T][Hq][D] (written; every row of a prompt)
 *   scale        softmax scale (1/sqrt(D) for the model)
 *   B            1 .. PA_MAX_PREFILL_BATCH; T total rows, 0 .. PA_MAX_PREFILL_ROWS
 *   weights      how the softmax weights meet V (scores, maxima and sums are FP32):
 *     PA_PREFILL_WEIGHTS_BF16X2  each weight as a bf16 pair (high part and
 *                remainder, within 2^-16 relative) times bf16 V: two MFMAs.
 *     PA_PREFILL_WEIGHTS_FP16    each weight rounded to fp16 (2^-11), V converted
 *                to fp16 (exact for |v| in [2^-17, 65504]; smaller values to
 *                within 2^-25; larger ones overflow), the row sum taken over the
 *                rounded weights: one MFMA; the error of an output is at most
 *                about 2^-10 times the spread of the V values it averages.
 * Inputs are expected finite: a non-finite value in one prompt's V can reach
 * rows of a neighbouring prompt that share its 16-row group.
 * cu_tokens breaking the rules above gives unspecified output but no access
 * outside q, k, v, out and cu_tokens[0 .. B].
 * Returns PA_OK, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_NULL, PA_ERR_ALIGN
 * or PA_ERR_LAUNCH; nothing is launched for T == 0.
 */
int pa_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu_tokens, int32_t B,
               int64_t T, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t weights, float* out,
               hipStream_t stream);

/*
 * Bytes of workspace pa_decode and pa_append_decode need for these sizes
 * (partition_tokens = 0: automatic split size).  Returns 0 for invalid sizes;
 * the calls report those.  ([README] feature list, persistent scratch buffers
 * item: scratch is sized once up front and reused across steps, rather than
 * allocated per call; this library never allocates, the caller owns the
 * buffer and can keep one per stream for the whole run.)
 */
size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_blocks,
                                 int32_t partition_tokens);

/* The partition_tokens value that selects the automatic split size (0). */
int32_t pa_default_partition_tokens(void);

/*
 * pa_decode - batched paged decode attention for one layer.
 * ([README] paged decode attention item: every query head streams its
 * sequence's cached pages with an FP32 online softmax and accumulates V,
 * with no contiguous gather and no stored scores; [NF].)
 *
 *   out[b][h][:] = sum_{t < L} softmax_t(scale * q[b][h] . K_t[g]) V_t[g],
 *   L = seq_lens[b], g = h / (Hq/Hkv), K_t / V_t read through block_table[b].
 *
 *   q            bf16 [B][Hq][D] (already position-encoded)
 *   out          fp32 [B][Hq][D]; rows of sequences with L == 0 are set to 0
 *   scale        softmax scale (1/sqrt(D) for the model)
 *   partition_tokens  split size in tokens, a multiple of 16; values above
 *                2048 act as 2048 (a split holds at most 128 pages).  So a
 *                value >= 16 * max_blocks gives every sequence a single pass
 *                only while max_blocks <= 128 (the 2048-token context of the
 *                pages' model); a longer table row still gets
 *                ceil(L / 2048) splits.  A sequence of L tokens (npages = ceil(L/16)
 *                pages) is processed as S_b = ceil(npages / pp) splits with
 *                pp = partition_tokens / 16 pages; split s takes the pages
 *                s, s + S_b, s + 2 S_b, ...  With partition_tokens > 0 the splits
 *                of a sequence depend only on its own length, so its output is
 *                bit-identical whatever else is in the batch.  With 0
 *                (automatic) pp = clamp(ceil(total pages of the batch / n), m,
 *                128) with n = 192 when every sequence has the same page count,
 *                otherwise n = 240 when total pages >= 8 B and 384 below, and
 *                m = 4 for B <= 64, 8 above (the
 *                smallest split): large batches get few, long splits and
 *                small or skewed batches get more; results then may differ in
 *                rounding between batches.  When S_b > 1 the splits' partial
 *                states are merged inside the same launch.
 *   B            at most PA_MAX_DECODE_BATCH (the work plan lives in LDS).
 *   workspace    device buffer of at least
 *                pa_decode_workspace_bytes(B, Hq, D, max_blocks, partition_tokens)
 *                bytes, zero-filled before its first use.  It holds the split
 *                partials (part_o, part_m, part_l in the layout pa_merge takes,
 *                with S = ceil(max_blocks / smallest split in pages)), one int32
 *                completion counter per (sequence, KV head) and a work-queue
 *                counter; the counters are back at zero when the call's work
 *                completes, so the buffer can be reused without clearing.  Calls
 *                that overlap in time must not share a workspace.  Splits are
 *                combined inside the same kernel, for each KV head by the last
 *                wave of the sequence's splits to finish it.
 * Arithmetic: QK^T products of BF16 values are exact in FP32 and summed in
 * FP32; softmax and accumulation are FP32; the exponentials are base 2 with
 * log2(e) folded into the scale.
 */
int pa_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
              const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, float scale,
              float* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages,
              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/*
 * pa_append_decode - pa_append followed by pa_decode, in one launch.
 * ([README] KV page pool item and paged decode attention item: the step
 * appends the new token at its absolute position, then attends over the
 * sequence's pages including it.)
 *
 * Arguments mean what they mean for pa_append and pa_decode; the pools are
 * written (the row of position L-1 of every sequence with L >= 1, as a bit
 * copy of k_new / v_new) and out is computed over positions 0..L-1 with that
 * row.  The pools and out end up bit-identical to pa_append followed by
 * pa_decode with the same arguments.
 */
int pa_append_decode(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                     uint16_t* v_pool, const uint16_t* q, const int32_t* block_table,
                     int32_t max_blocks, const int32_t* seq_lens, float scale, float* out, int32_t B,
                     int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, int32_t partition_tokens,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_plan - the work plan of one decode step, built once and read by
 * every layer's pa_decode_planned launch of that step.
 * ([README] batched decode item: each step packs one token of every active
 * sequence, with separate page mappings and attention lengths per sequence;
 * the lengths are the same for all layers of the step, so the split of each
 * sequence into work items and their assignment to workgroups are too.)
 *
 *   seq_lens     int32 [B] (device), the lengths after this step's append
 *   plan         device buffer of at least pa_decode_plan_bytes(B, max_blocks,
 *                partition_tokens) bytes, written by one small kernel on stream
 *   partition_tokens  as for pa_decode (0: automatic); the splits are exactly
 *                those pa_decode makes for the same lengths and value
 * The plan holds the lengths, the split of every sequence and the order of
 * the (sequence, split) items: each workgroup of the decode launch takes item
 * w first and claims the rest through the workspace's queue counter.  Long
 * items (8 pages or more on average) are ordered by pages, longest first;
 * shorter ones keep sequence order, multi-split sequences first.  It must be
 * rebuilt whenever seq_lens changes; a plan used with lengths other than those
 * it was built from reads the block-table entries its own lengths reach.  Returns PA_OK, PA_ERR_SHAPE, PA_ERR_NULL, PA_ERR_ALIGN,
 * PA_ERR_WORKSPACE (plan too small) or PA_ERR_LAUNCH; B == 0 does nothing.
 */
size_t pa_decode_plan_bytes(int32_t B, int32_t max_blocks, int32_t partition_tokens);
int pa_decode_plan(const int32_t* seq_lens, int32_t B, int32_t max_blocks, int32_t partition_tokens, void* plan,
                   size_t plan_bytes, hipStream_t stream);

/*
 * pa_decode_planned - pa_decode, pa_append_decode or pa_rope_append_decode
 * (by which of k_new / v_new / cos_sin are given) with the work items taken
 * from a plan of pa_decode_plan instead of being planned inside the launch.
 * ([README] paged decode attention item, KV page pool item and feature list,
 * as for those calls.)
 *
 *   k_new, v_new  NULL (attention only: the pools are read, not written), or
 *                 both given: the append of pa_append_decode first
 *   cos_sin, max_pos  NULL / 0, or RoPE of q and the new key as in
 *                 pa_rope_append_decode (needs k_new, v_new; max_pos >= 16 *
 *                 max_blocks)
 *   plan, plan_bytes  a plan pa_decode_plan wrote for this step's lengths with
 *                 the same B, max_blocks and partition_tokens, on a device with
 *                 the same compute-unit count; the lengths come from it (no
 *                 seq_lens argument)
 *   workspace    as for pa_decode (the same size for the same partition_tokens)
 *   other arguments as for pa_append_decode.
 * out and the pools are bit-identical to the unplanned call on the same
 * lengths.  If the plan's header does not match B, max_blocks,
 * partition_tokens and the launch, every element of out is set to NaN.
 */
int pa_decode_planned(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const float* cos_sin,
                      int32_t max_pos, uint16_t* k_pool, uint16_t* v_pool, const int32_t* block_table,
                      int32_t max_blocks, float scale, float* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                      int64_t num_pages, int32_t partition_tokens, const void* plan, size_t plan_bytes,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_append_decode_noalloc - pa_append_decode for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses that
 * forbid allocation.  It takes no workspace and allocates nothing: the split
 * partials, counters and queue live in a device array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from the first call on that GPU until the process ends.
 *
 * Arguments, results and bit-identity are those of pa_append_decode.  Each call
 * first clears the counters it uses (a kernel on `stream`, no memset), then
 * launches the decode.  Limit: the workspace pa_decode_workspace_bytes(B, Hq,
 * D, max_blocks, partition_tokens) would report must fit in the array, else
 * PA_ERR_SCRATCH is returned before anything touches the device (64 MiB holds
 * B = 64 at 128 table entries under the automatic split, B = 256 at 128
 * entries with splits of 128 tokens or more, and any batch with
 * partition_tokens >= 16 * max_blocks up to 2048 tokens).  Every call on a
 * GPU shares that GPU's array and it keeps the last call's contents: calls
 * that overlap in time on one GPU (two streams, two threads, two captured
 * graphs replayed concurrently) race and give wrong results; issue them on one
 * stream or order them with events.
 */
int pa_append_decode_noalloc(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                             uint16_t* v_pool, const uint16_t* q, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* seq_lens, float scale, float* out, int32_t B,
                             int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, int32_t partition_tokens,
                             hipStream_t stream);

/*
 * pa_merge - combine split partial states into the attention output.
 * (Split-K over page ranges is this library's own; it is exact because the
 * log-sum-exp merge of softmax partial states is an identity.)
 *
 *   part_o  fp32 [B][Hq][S][D]: split s's output, already divided by its l
 *   part_m  fp32 [B][Hq][S]: maximum over the split of x_t = scale*log2(e)*(q.K_t)
 *           (a base-2 logit)
 *   part_l  fp32 [B][Hq][S]: sum over the split of 2^(x_t - part_m)
 *   A state kept with natural-log maxima (m_e = max of scale*(q.K_t),
 *   l = sum of e^(scale*(q.K_t) - m_e)) converts by part_m = m_e * log2(e);
 *   l and o are the same in both bases, since 2^(x_t - part_m) = e^(s_t - m_e).
 *   seq_lens int32 [B] or NULL.  With seq_lens, split s of sequence b is live
 *           iff s*partition_tokens < seq_lens[b] (the splits pa_decode makes:
 *           partition_tokens above 2048 act as 2048 here too) and sequences
 *           with L == 0 get zeros; with NULL every split is live.
 *   A split's token set does not matter to the merge: any partition of a
 *   sequence's tokens into splits gives the same result.
 *   out     fp32 [B][Hq][D]
 *   out = sum_s w_s o_s / sum_s w_s,  w_s = l_s 2^(m_s - max_s m_s), over live
 *   splits with l_s > 0; zero if there is none.
 */
int pa_merge(const float* part_o, const float* part_m, const float* part_l,
             const int32_t* seq_lens, int32_t partition_tokens, float* out, int32_t B, int32_t Hq,
             int32_t D, int32_t S, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
