/*
 * fdllm.h -- C ABI of the MI355X (gfx950) library for the per-layer hot path of
 * one Flash-dLLM decoding step.
 *
 * Pages cited (public summaries of one preprint):
 *   [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
 *        Memory-Efficient Diffusion LLMs", ai4snews.wisdomeyes.cn summary,
 *        paragraphs 1-5.
 *   [P2] arXiv abstract page of the same preprint.
 *
 * Conventions for every entry point
 *   - Buffer arguments are DEVICE pointers owned by the caller (for example
 *     torch.Tensor.data_ptr()).  The library never allocates, frees or keeps
 *     caller memory; scratch space comes from the caller's `workspace`.
 *   - Struct arguments (fdl_kv_cache) are HOST structs read during the call only.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *     asynchronous and ordered on that stream; nothing synchronises the host.
 *     Inputs must stay alive, and outputs are valid, once the stream reaches
 *     the end of the call.
 *   - Calls on different streams must use different output/workspace buffers.
 *   - bf16 = IEEE bfloat16 bit patterns, round-to-nearest-even when produced.
 *   - Return value: FDL_OK, or an error code.  Size, pointer and shape checks
 *     happen on the host before any launch; on error nothing is launched.
 *     Index contents of device arrays (positions, slots, block ids, lengths)
 *     are not read by the host: values out of range are undefined behaviour,
 *     as for any paged-attention kernel; the caller validates them.
 *   - With FDL_DEBUG=1 in the environment (read at every call), the calls that
 *     index the cache (flash_cache_step, flash_cache_step_unfused,
 *     scheduled_attention, flash_cache_attention_step) first synchronise their
 *     stream and check those arrays on the host: cu_rows starts at 0, never
 *     decreases and ends at most at num_rows; active rows have positions >= 0
 *     and logical slots inside their block-table row; every block id a row
 *     writes or a visible slot reads lies in [0, num_blocks); lengths are
 *     >= 0; no physical slot is written by two rows; no sequence has more
 *     rows than max_rows_per_seq; two-view descriptors are non-negative and
 *     meet their stated inequalities.  A violation returns FDL_EINVAL with
 *     nothing launched (a failed copy, FDL_EHIP).
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {32, 64, 128, 256};
 * hidden a multiple of 128 and at most 32768; num_heads * head_dim <= 16384;
 * at most 1024 cache pages per sequence (max_kv_len <= 1024 * block_size).
 */
#ifndef FDLLM_H
#define FDLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FDL_OK = 0,
  FDL_EINVAL = 1,       /* null pointer, negative or inconsistent size */
  FDL_EUNSUPPORTED = 2, /* shape outside the supported set above */
  FDL_EWORKSPACE = 3,   /* workspace smaller than fdl_attention_workspace_bytes() */
  FDL_EHIP = 4,         /* a HIP launch failed; see fdl_last_hip_error() */
  FDL_ESCRATCH = 5      /* the sizes need more scratch than the static buffer holds */
};

/* Paged KV cache of one layer [P4 para 1: keys and values written directly into
 * the KV cache; a block table maps each sequence's logical blocks].
 * Pools are bf16 [num_blocks][num_heads][block_size][head_dim]: the keys of one
 * head inside one page are contiguous (block_size * head_dim elements).
 * Logical slot s of sequence b is physical block block_table[b*max_blocks_per_seq
 * + s / block_size], offset s % block_size; its "physical slot" number is
 * block * block_size + offset.  Entries past ceil(kv_len / block_size) of a
 * sequence are never read. */
typedef struct fdl_kv_cache {
  int32_t num_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  void *k_cache;              /* device bf16 pool (written by flash_cache_step) */
  void *v_cache;              /* device bf16 pool */
  const int32_t *block_table; /* device int32 [batch][max_blocks_per_seq] */
} fdl_kv_cache;

/* Two-view (Flash-Verify) descriptor of one sequence [P4 para 3].
 * window_len == 0: plain sequence; every row attends to every slot < kv_len.
 * Otherwise the window's own slots window_start .. window_start+window_len-1
 * hold the MASK view, the DRAFT view's keys sit at slots draft_slot_start ..
 * draft_slot_start+window_len-1 (same rotary positions), and the sequence's
 * rows are window_len draft rows followed by mask rows.  Draft row i sees the
 * context (slots < draft_slot_start outside the window) and draft slots
 * draft_slot_start .. draft_slot_start+i; every later row (mask view) sees all
 * slots < draft_slot_start.  Requires window_start + window_len <=
 * draft_slot_start and draft_slot_start + window_len <= kv_len. */
typedef struct fdl_two_view {
  int32_t window_start;
  int32_t window_len;
  int32_t draft_slot_start;
} fdl_two_view;

/* Flash-Cache [P4 para 1; P4 para 2 for which rows are active]: for the
 * num_rows active rows (sliding unmasking window plus tracked rows of every
 * sequence), Y = X . W_qkv in fp32, rotary embedding of the Q and K parts at
 * each row's position, rounding to bf16, K and V rows written straight into the
 * paged cache at the row's slot, Q written to q_out.  One fused launch: the
 * projections never make an HBM round trip.
 *   x          device bf16 [num_rows][hidden]
 *   w_qkv      device bf16 [3*H*D][hidden]: output feature n is row n (the
 *              nn.Linear weight layout); features [0,HD) are Q, [HD,2HD) K,
 *              [2HD,3HD) V; head h owns features h*D .. h*D+D-1 of each part.
 *   cu_rows    device int32 [batch+1]; rows of sequence b are cu_rows[b] ..
 *              cu_rows[b+1]-1 (non-decreasing, cu_rows[0] == 0,
 *              cu_rows[batch] <= num_rows).  Rows cu_rows[batch] .. num_rows-1
 *              are inactive: nothing is read from positions/slots or written
 *              to q_out, slot_mapping_out or the cache for them.  num_rows is
 *              then a capacity, so a row count chosen on the device (see
 *              decode_plan) needs no host round trip.
 *   positions  device int32 [num_rows], rotary position (0-based) of each row.
 *   slots      device int32 [num_rows], logical cache slot of each row; slots
 *              of one call must map to distinct physical slots.
 *   rope_base  rotary base; pairs (i, i + D/2), angle position*base^(-2i/D).
 *   q_out      device bf16 [num_rows][H][D]
 *   slot_mapping_out  device int64 [num_rows] physical slot of each row, or NULL.
 *   workspace  device scratch of fdl_flash_cache_workspace_bytes(...) bytes
 *              (no initialisation needed); NULL when that is 0.
 * x, w_qkv, q_out and both cache pools must be 16-byte aligned (they are read
 * and written in 16-byte pieces); otherwise FDL_EINVAL, nothing launched.
 * num_rows == 0 or batch == 0 is a no-op.  Output bits do not depend on the
 * order in which workgroups finish: partial sums are added in a fixed order. */
int flash_cache_step(const fdl_kv_cache *cache, const void *x, int32_t hidden,
                     const void *w_qkv, int32_t batch, int32_t num_rows,
                     const int32_t *cu_rows, const int32_t *positions,
                     const int32_t *slots, float rope_base, void *q_out,
                     int64_t *slot_mapping_out, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Ablation of Flash-Cache [P4 para 1: the prior practice of separate kernel
 * launches per layer that move intermediates to and from HBM]: the same
 * results as flash_cache_step (bitwise: the same projection kernels and the
 * same rotation/rounding helper), computed as three launches -- the
 * projection writes fp32 Y [num_rows][3HD] to the workspace, a rotary kernel
 * writes bf16 Q to q_out and bf16 K, V rows to workspace staging, and a
 * scatter kernel copies them into the paged cache.  Same arguments and error
 * behaviour as flash_cache_step; the workspace must hold
 * fdl_flash_cache_unfused_workspace_bytes(...) bytes. */
int flash_cache_step_unfused(const fdl_kv_cache *cache, const void *x, int32_t hidden,
                             const void *w_qkv, int32_t batch, int32_t num_rows,
                             const int32_t *cu_rows, const int32_t *positions,
                             const int32_t *slots, float rope_base, void *q_out,
                             int64_t *slot_mapping_out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Workspace bytes flash_cache_step_unfused needs (0 for invalid sizes). */
size_t fdl_flash_cache_unfused_workspace_bytes(int32_t num_rows, int32_t hidden,
                                               int32_t num_heads, int32_t head_dim);

/* Workspace bytes flash_cache_step needs for these sizes (0: none; then
 * workspace may be NULL).  It holds the fp32 partial sums of a reduction split
 * across workgroups; two calls that may run at the same time must not share
 * a workspace. */
size_t fdl_flash_cache_workspace_bytes(int32_t num_rows, int32_t hidden,
                                       int32_t num_heads, int32_t head_dim);

/* Scheduled attention [P4 para 1: block-table scheduling over the ragged
 * lengths of a batch; P4 para 3: two-view mask] plus, when `mass` is not NULL,
 * the attention mass that ranks the most-attended keys [P4 para 2].
 * For sequence b, head h and row r: P = softmax(scale * q_r . k_j) over the
 * visible slots j < kv_len[b] (see fdl_two_view), out_r = sum_j P_j v_j.
 *   q          device bf16 [num_rows][H][D] (as written by flash_cache_step)
 *   cu_rows    as for flash_cache_step: rows cu_rows[batch] .. num_rows-1 are
 *              inactive and their `out` rows are not written.
 *   kv_len     device int32 [batch]; max_kv_len >= every kv_len[b] (host bound;
 *              a larger kv_len[b] is read as max_kv_len).
 *   max_rows_per_seq  host upper bound on cu_rows[b+1]-cu_rows[b].
 *   Cache slots at or past kv_len[b] are never used, whatever they hold (NaN
 *   included), even when they share a page with visible slots.
 *   views      device fdl_two_view [batch], or NULL (all sequences plain).
 *   softmax_scale  0 selects 1/sqrt(D).
 *   out        device fp32 [num_rows][H][D]; a row that sees no key gets 0.
 *   mass       device fp32 [batch][mass_stride] or NULL:
 *              mass[b][j] = sum over heads and rows of P, for j < kv_len[b];
 *              entries kv_len[b] <= j < mass_stride are set to 0.  The sum runs
 *              in a fixed order: results are bitwise reproducible.
 *   mass_stride >= max_kv_len when mass is given.
 *   workspace  device scratch of at least fdl_attention_workspace_bytes(...)
 *              bytes (same arguments); contents need no initialisation.  On
 *              FDL_PATH_SPLIT_MASS_EXCHANGE (fdl_attention_path) with a cache
 *              past 1024 keys, the splits of a sequence wait for each other's
 *              row statistics through counters the call clears itself at its
 *              start; the int32 at byte 4 is then an error word that becomes
 *              1 if such a wait ever timed out (it never should: every wait is
 *              for a running workgroup) and stays 1 until the caller clears
 *              it; the results of such a call are invalid.  Calls that share a
 *              workspace must not run at the same time. */
int scheduled_attention(const fdl_kv_cache *cache, const void *q, int32_t batch,
                        int32_t num_rows, const int32_t *cu_rows,
                        const int32_t *kv_len, int32_t max_kv_len,
                        int32_t max_rows_per_seq, const fdl_two_view *views,
                        float softmax_scale, float *out, float *mass,
                        int32_t mass_stride, void *workspace,
                        size_t workspace_bytes, void *stream);

/* scheduled_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, semantics and results (the same kernels) as
 * scheduled_attention, without the workspace: its scratch is one static
 * device buffer of fdl_static_scratch_bytes() bytes (16 MiB) per GPU, held by
 * the library until the process ends; its address is looked up once per
 * device (the first call on it) and no call allocates or frees memory.
 *   Sizes whose fdl_attention_workspace_bytes(...) exceeds that buffer are
 *   refused with FDL_ESCRATCH before anything is launched.
 *   The buffer belongs to the current device; `stream` must be a stream of
 *   that device.  Every call on a GPU uses the same buffer, which keeps the
 *   previous call's contents (the call clears what must start at zero):
 *   calls that overlap on one GPU (other streams, other host threads) race
 *   and must not be issued.  The error word of the exchange path (see
 *   scheduled_attention) is byte 4 of the buffer. */
int scheduled_attention_static(const fdl_kv_cache *cache, const void *q, int32_t batch,
                               int32_t num_rows, const int32_t *cu_rows,
                               const int32_t *kv_len, int32_t max_kv_len,
                               int32_t max_rows_per_seq, const fdl_two_view *views,
                               float softmax_scale, float *out, float *mass,
                               int32_t mass_stride, void *stream);

/* Size in bytes of scheduled_attention_static's static scratch buffer. */
size_t fdl_static_scratch_bytes(void);

/* The kernels scheduled_attention uses for these sizes (mass_stride 0 = no
 * mass); the results agree on every path within float rounding:
 *   FDL_PATH_ROW_GROUPS  one workgroup per (sequence, head, 16 rows) over the
 *       whole cache (small grids, caches up to 1024 keys, mass asked for);
 *   FDL_PATH_SPLIT  (sequence, 64 rows, head, KV split) workgroups with a
 *       fixed-order merge of the splits (no mass);
 *   FDL_PATH_SPLIT_MASS_EXCHANGE  (sequence, 64 rows, head, 1024-key split)
 *       workgroups keeping their scores on chip; the splits of a longer cache
 *       exchange row statistics, so keys are read once;
 *   FDL_PATH_SPLIT_MASS_REREAD  one workgroup per (sequence, 64 rows, head)
 *       whose mass is a second, last-first pass over K right after the first
 *       (caches past 1024 keys with enough sequences x heads to fill the GPU).
 * Returns 0 for invalid sizes. */
enum {
  FDL_PATH_ROW_GROUPS = 1,
  FDL_PATH_SPLIT = 2,
  FDL_PATH_SPLIT_MASS_EXCHANGE = 3,
  FDL_PATH_SPLIT_MASS_REREAD = 4
};
int fdl_attention_path(int32_t batch, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                       int32_t max_kv_len, int32_t max_rows_per_seq, int32_t mass_stride);

/* Workspace bytes scheduled_attention needs for these sizes (mass_stride 0 =
 * no mass).  Returns 0 for invalid sizes. */
size_t fdl_attention_workspace_bytes(int32_t batch, int32_t num_rows,
                                     int32_t num_heads, int32_t head_dim,
                                     int32_t max_kv_len, int32_t max_rows_per_seq,
                                     int32_t mass_stride);

/* Next tracking set [P4 para 2: a fixed budget of most-attended tokens]:
 * per sequence the topb keys j < kv_len[b] with the largest mass[b][j]; equal
 * masses go to the lower index.  Written as a set in ascending index order to
 * idx_out (device int32 [batch][topb]); when kv_len[b] < topb the tail is -1.
 * A kv_len[b] larger than mass_stride is read as mass_stride.
 * mass values must be non-negative and not NaN (attention masses are). */
int track_topb(const float *mass, int32_t mass_stride, const int32_t *kv_len,
               int32_t batch, int32_t topb, int32_t *idx_out, void *stream);

/* Flash-Verify acceptance [P4 para 3]: per sequence, the length of the longest
 * prefix of positions k = 0, 1, ... where draft_tok == mask_tok and conf is
 * strictly greater than threshold; the scan stops at the first failure.
 *   draft_tok, mask_tok  device int32 [batch][window]
 *   conf                 device fp32 [batch][window] (NaN fails)
 *   accept_len_out       device int32 [batch]
 * window == 0 gives 0 for every sequence. */
int verify_accept(const int32_t *draft_tok, const int32_t *mask_tok,
                  const float *conf, int32_t batch, int32_t window,
                  float threshold, int32_t *accept_len_out, void *stream);

/* One call for the step [P4 para 1: the fused cache kernel combined with
 * scheduled attention]: flash_cache_step followed by scheduled_attention with
 * the mass, the two calls' kernels launched back to back on `stream` (on this
 * part a kernel boundary is the cheapest hand-off of Q and the written K/V
 * between XCDs: a single persistent launch, and a projection overlapped with
 * the cached keys' attention on a second stream, were both measured slower).
 * Arguments as for those two calls (the attention reads the q_out this call
 * writes); mass must not be NULL.  Results are bitwise those of the two
 * separate calls.  Every shape the two calls take is supported.
 *   workspace  fdl_fused_step_workspace_bytes(...) bytes (the same workspace
 *              also serves flash_cache_attention_step_single_launch); contents
 *              need no initialisation.  The attention's workspace starts at
 *              byte 4096, so its error word (see scheduled_attention) is the
 *              int32 at byte 4100. */
int flash_cache_attention_step(const fdl_kv_cache *cache, const void *x, int32_t hidden,
                               const void *w_qkv, int32_t batch, int32_t num_rows,
                               const int32_t *cu_rows, const int32_t *positions,
                               const int32_t *slots, float rope_base, void *q_out,
                               int64_t *slot_mapping_out, const int32_t *kv_len,
                               int32_t max_kv_len, int32_t max_rows_per_seq,
                               const fdl_two_view *views, float softmax_scale, float *out,
                               float *mass, int32_t mass_stride, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Single-launch step [P4 para 1: the fused cache kernel combined with
 * scheduled attention; P4 para 3: the verify mask inside the fused kernel]:
 * flash_cache_step followed by scheduled_attention with the mass, as one
 * persistent launch (an alternative form of flash_cache_attention_step, kept
 * for comparison: on this part it is slower than the back-to-back kernels).
 * Arguments as for flash_cache_attention_step.
 * Items are dealt to the XCDs by head (XCD x owns heads x, x + 8, ...): each
 * XCD's queue holds the projection items of its heads' Q, K and V features,
 * then the row-group attention items of those heads.  A workgroup takes items
 * from the queue of the XCD it runs on (read from the hardware), so a head's
 * projection hands Q and the written K/V to its attention through that XCD's
 * L2: a per-head count, no L2 write-back.  An attention item starts once its
 * own head is projected; the mass items (a sum over every head) start after
 * each XCD has written its L2 back once.  An item only waits for items with
 * lower tickets, held by running workgroups, so the ordinary launch needs no
 * co-residency guarantee.  Results agree with the two separate calls' (each
 * item runs their workgroup code): bitwise with the tiled projection (more
 * than 64 rows); with the split-K projection the column groups are formed per
 * XCD, so Q, K and V may differ in the last bit (another order of the fp32
 * sums).  Every call gives bitwise the same results as the last.
 *   workspace  fdl_fused_step_workspace_bytes(...) bytes.  Its first 4096
 *              bytes hold the counters, the tickets and an error word: they
 *              must be zero before the first call (for example a zero-filled
 *              allocation, made in stream order before the call); each call
 *              leaves the counters zero.  The error word (int32 at byte 12)
 *              becomes 1 if a wait ever timed out (it never should: every
 *              wait is for a running workgroup); results are then invalid,
 *              and the word stays set until the caller clears it.  Calls
 *              sharing a workspace must not run at the same time.
 * Supported: the shapes whose separate calls take a one-launch projection (no
 * split reduction) and the row-group attention path (few sequences x heads,
 * caches up to 1024 keys), with at most 1004 heads; otherwise
 * FDL_EUNSUPPORTED and nothing launched.  The part is taken to have 8 XCDs
 * (XCC_ID 0..7); a device with fewer runs no item of the missing XCDs' queues,
 * and the mass wait then times out and sets the error word. */
int flash_cache_attention_step_single_launch(
    const fdl_kv_cache *cache, const void *x, int32_t hidden, const void *w_qkv, int32_t batch,
    int32_t num_rows, const int32_t *cu_rows, const int32_t *positions, const int32_t *slots,
    float rope_base, void *q_out, int64_t *slot_mapping_out, const int32_t *kv_len,
    int32_t max_kv_len, int32_t max_rows_per_seq, const fdl_two_view *views, float softmax_scale,
    float *out, float *mass, int32_t mass_stride, void *workspace, size_t workspace_bytes,
    void *stream);

/* Workspace bytes flash_cache_attention_step and
 * flash_cache_attention_step_single_launch need, for any hidden size (0 for
 * invalid sizes; mass_stride > 0). */
size_t fdl_fused_step_workspace_bytes(int32_t batch, int32_t num_rows, int32_t num_heads,
                                      int32_t head_dim, int32_t max_kv_len,
                                      int32_t max_rows_per_seq, int32_t mass_stride);

/* Planning step of a multi-step decoding loop [P4 para 2: each step's query
 * rows are a sliding unmasking window plus a fixed budget of the most-attended
 * tokens; P4 para 1: caching (refresh) and update stages alternate within a
 * batch; P4 para 3: accepted tokens are committed in causal order].  Runs on
 * the device, so a loop of steps needs no host round trip.  Per sequence b,
 * with L = kv_len[b] and f = frontier[b] clamped to [0, L] (the first
 * position not yet committed):
 *   1. step > 0: f += max(1, min(accept_len[b], window_len)), capped at L
 *      (at least one token per step; accept_len < 0 reads as 0).
 *   2. f == L: the sequence is finished and gets no rows (stage 2).
 *   3. Stage: refresh (1) when refresh_period > 0 and (step + b) %
 *      refresh_period == 0, else update (0).  The window is [w0, min(w0 +
 *      window_len, L)) with w0 = f (update) or the block_size boundary at or
 *      below f (refresh).
 *   4. Tracked rows: entries of tracked[b] kept when in [0, L), outside the
 *      window and above every entry kept before them (a track_topb result is
 *      ascending; this also drops repeats and -1 padding).
 *   5. Rows: the window positions ascending, then the kept tracked entries;
 *      slot = position.
 *   kv_len       device int32 [batch]
 *   tracked      device int32 [batch][topb]: the previous step's track_topb
 *                output (the caller's initial set at step 0); may be NULL when
 *                topb == 0.
 *   accept_len   device int32 [batch]: the previous step's verify_accept
 *                output; not read at step 0 (may be NULL then).
 *   frontier     device int32 [batch], read and then overwritten with the
 *                new f.
 *   cu_rows_out  device int32 [batch+1]; positions_out, slots_out device int32
 *                [row_capacity]; stage_out device int32 [batch] or NULL.
 *   row_capacity >= batch * (window_len + topb), which bounds every plan.
 * batch <= 4096 (FDL_EUNSUPPORTED above); window_len >= 1, block_size >= 1,
 * refresh_period >= 0, step >= 0, topb >= 0 (FDL_EINVAL otherwise).  One
 * workgroup plans the batch. */
int decode_plan(int32_t batch, const int32_t *kv_len, int32_t window_len,
                int32_t block_size, int32_t refresh_period, int32_t step,
                const int32_t *tracked, int32_t topb, const int32_t *accept_len,
                int32_t *frontier, int32_t *cu_rows_out, int32_t *positions_out,
                int32_t *slots_out, int32_t *stage_out, int32_t row_capacity,
                void *stream);

/* Hidden states of the planned rows for a loop whose model is not given (the
 * input rows of flash_cache_step): row r of sequence b at position p copies
 * hidden_committed[b][p] when p < frontier[b] (a committed token), else
 * hidden_masked[b][p] (a still-masked position).
 *   cu_rows, positions, frontier  as written by decode_plan
 *   hidden_committed, hidden_masked  device bf16 [batch][max_len][hidden],
 *                16-byte aligned; positions are clamped to [0, max_len).
 *   x_out        device bf16 [row_capacity][hidden], 16-byte aligned; rows
 *                cu_rows[batch] .. row_capacity-1 are not written.
 * hidden must be a positive multiple of 8. */
int gather_hidden(int32_t batch, int32_t row_capacity, const int32_t *cu_rows,
                  const int32_t *positions, const int32_t *frontier,
                  const void *hidden_committed, const void *hidden_masked,
                  int32_t max_len, int32_t hidden, void *x_out, void *stream);

/* Mask-view confidence producer [P4 para 3: a position is accepted when the
 * two views agree and the mask-view confidence exceeds the threshold].
 * Reading: the LM head maps each row's final hidden state to vocabulary
 * logits z = h . W^T (bf16 inputs, fp32 accumulate); the row's token is the
 * argmax (equal logits go to the lower id) and its confidence the softmax
 * probability of that token, 1 / sum_v exp(z_v - z_max).  The logits never
 * reach memory.  Applied to the draft rows it gives the draft tokens, to the
 * mask rows the tokens and confidences that verify_accept compares.
 *   hidden_states  device bf16 [rows][hidden]
 *   w_lm           device bf16 [vocab][hidden] (the nn.Linear weight; no bias)
 *   token_out      device int32 [rows]; conf_out device fp32 [rows]
 *   workspace      device scratch of fdl_lm_head_workspace_bytes(rows, vocab)
 *                  bytes (per-tile partial maxima, sums and ids).
 * hidden must be a multiple of 32 and at most 65536 (FDL_EUNSUPPORTED);
 * rows == 0 is a no-op.  Results are bitwise reproducible (fixed-order
 * reductions). */
int lm_head_confidence(const void *hidden_states, const void *w_lm, int32_t rows,
                       int32_t vocab, int32_t hidden, int32_t *token_out,
                       float *conf_out, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Workspace bytes lm_head_confidence needs (0 for invalid sizes). */
size_t fdl_lm_head_workspace_bytes(int32_t rows, int32_t vocab);

/* Text for a status code (static storage). */
const char *fdl_status_string(int status);

/* hipError_t of the most recent FDL_EHIP on this host thread (0 if none). */
int fdl_last_hip_error(void);

/* Library version string. */
const char *fdl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FDLLM_H */
