/*
 * lora_mi355x.h - C ABI of the MI355X (gfx950) multi-LoRA shrink/expand path.
 *
 * One batch of tokens, each tagged with an adapter id (or -1 for none), is
 * projected through per-adapter low-rank weights:
 *
 *   shrink:  buf[s][t][0:r]            = scale * x[t][:] . A_s[l]^T
 *   expand:  y[t][off_s : off_s + n_s] += buf[s][t][:] . B_s[l]^T
 *
 * with l = token_lora_mapping[t] and off_s = n_0 + ... + n_{s-1}.  The batch is
 * not grouped by adapter; a metadata step groups it on the device first.
 *   - vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1": the summary names
 *     the shrink and expand kernels; "Why do we need a new set of kernels"
 *     explains that V1 batches are not grouped by LoRA id, so the kernels are
 *     handed the token -> LoRA mapping and load the tokens it selects; "Kernel
 *     Code Change" item 1 asks for a launch grid that CUDA graphs can capture,
 *     item 2 for the gather of the input tokens.
 *   - MLC-LLM issue "[Tracking] Multi-LoRA Serving", Overview: Punica's one-launch
 *     kernel over a batch split into per-request row segments, each multiplied by
 *     its own low-rank weights.
 *   - vLLM PR #14626 "[Kernel] LoRA - Enable CUDAGraphs for V1", review
 *     comments: the LoRA index buffers are static, sized by the maximum token
 *     count, captured with their shapes; the graph's pad region is not cleared,
 *     so inputs must never be updated in place.
 *
 * Conventions shared by every entry point:
 *   - bf16 tensors are passed as raw uint16 bit patterns; fp32 as float.
 *   - Every pointer is a DEVICE pointer unless marked "host".  All memory is
 *     owned by the caller.  No call allocates, frees, synchronises or keeps
 *     state between calls; host arrays are read only during the call.
 *   - Every call enqueues one kernel on `stream` (lora_prepare_and_shrink and
 *     lora_fused_step: one or more, see there) and returns without waiting.  Launch grids depend
 *     only on the size arguments (max_tokens, max_loras, shapes), never on
 *     device data, so a sequence of calls can be
 *     captured once into a HIP graph and replayed.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid one returns LORA_ERR_INVALID_ARGUMENT and enqueues nothing.
 *   - Adapter ids outside [-1, max_loras) are device data and cannot raise an
 *     error without a synchronisation; they are treated as -1 (no adapter).
 *   - Inputs (x, A, B, the mapping) are never written.  Outputs are written only
 *     where stated; everything else is left untouched.
 *   - Calls that write the same buffers must be ordered on one stream.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARGUMENT = 1, /* a null pointer, a size out of range, a misaligned buffer */
  LORA_ERR_UNSUPPORTED = 2,      /* valid, but outside the shapes this library implements */
  LORA_ERR_LAUNCH = 3            /* the HIP runtime refused the launch */
} lora_status_t;

/* Largest supported values of the size arguments. */
#define LORA_MAX_LORAS 256     /* adapter slots */
#define LORA_MAX_SLICES 4      /* output slices per call (qkv: 3, gate_up: 2) */
#define LORA_MAX_SPLITS 64     /* hidden-dimension partitions of the shrink */

/* Tiles of the padded grouped order (see lora_meta_t): LORA_TILE positions
 * each, at most LORA_MAX_TILES(max_tokens, max_loras) of them. */
#define LORA_TILE 16
#define LORA_MAX_TILES(max_tokens, max_loras) \
  (((max_tokens) + LORA_TILE - 1) / LORA_TILE + (max_loras) + 1)

/*
 * Per-batch grouping of the tokens by adapter: the segment description that
 * shrink and expand read.  A host struct holding device pointers; the struct
 * itself is read only during a call.  One metadata result serves every LoRA
 * layer of the batch.
 *
 *   sorted_token_ids    int32 [max_tokens]: token indices grouped by adapter id
 *                       in ascending id order, tokens without an adapter
 *                       first, token order kept within a group (stable).
 *                       Entries [num_tokens, max_tokens) are never written.
 *   active_lora_ids     int32 [max_loras]: the adapter ids that occur in the
 *                       batch, ascending; unused slots hold -1.
 *   num_tokens_per_lora int32 [max_loras]: tokens per active slot; unused 0.
 *   lora_token_start    int32 [max_loras]: offset of the slot's first token in
 *                       sorted_token_ids; unused slots hold num_tokens.
 *   num_active          int32 [1]: number of active slots.
 *
 * The same grouping of the tokens that have an adapter, padded so that every
 * tile of LORA_TILE positions belongs to one adapter (the kernels read a
 * tile's token ids and its adapter at fixed addresses, in one round trip):
 *
 *   tile_token_ids      int32 [LORA_MAX_TILES * LORA_TILE]: the k-th active
 *                       slot's tokens (in sorted_token_ids order) from
 *                       position P_k = round_up(S_k + (LORA_TILE - 1) * k,
 *                       LORA_TILE), where S_k counts the tokens of the slots
 *                       before it; every other position below
 *                       num_tiles * LORA_TILE holds -1.  (The slack term makes
 *                       P_k a function of S_k and k alone, so each slot's
 *                       start is known without the other slots' sizes; it
 *                       leaves at most one empty tile between two slots.)
 *   tile_lora           int32 [LORA_MAX_TILES]: the adapter id of each tile
 *                       below num_tiles, or -1 for a tile of -1 entries.
 *   num_tiles           int32 [1]: tiles in use.
 *   Entries at or past num_tiles are never written.
 *
 * And one count of the batch as given (before grouping):
 *
 *   num_runs            int32 [1]: the number of maximal runs of consecutive
 *                       tokens (batch order) sharing one adapter id >= 0;
 *                       tokens without an adapter belong to no run.  Punica's
 *                       segment count for the batch as it arrives (MLC-LLM
 *                       issue, Overview).  Runs of at least a few tokens mean
 *                       that a tile of the grouped order holds neighbouring
 *                       rows of x and y; the expand picks its walk over the
 *                       tiles by it.
 */
typedef struct lora_meta {
  int32_t *sorted_token_ids;
  int32_t *active_lora_ids;
  int32_t *num_tokens_per_lora;
  int32_t *lora_token_start;
  int32_t *num_active;
  int32_t *tile_token_ids;
  int32_t *tile_lora;
  int32_t *num_tiles;
  int32_t *num_runs;
} lora_meta_t;

/*
 * lora_prepare_metadata - group the batch's tokens by adapter on the device.
 *
 * Defined by: vLLM PR #13096, "Why do we need a new set of kernels" (the
 * kernels must know which tokens map to which LoRA id) and "Kernel Code
 * Change" item 1 (graph-capturable launch grid); vLLM PR #14626 review
 * comments (static metadata buffers sized by the maximum token count); the
 * MLC-LLM issue's Overview (Punica's per-request segment vector).
 *
 *   token_lora_mapping  int32 [num_tokens], device; any value, ids outside
 *                       [-1, max_loras) count as -1.
 *   num_tokens          0 <= num_tokens <= max_tokens.
 *   max_tokens          capacity of sorted_token_ids, 1 <= max_tokens <= 2^24.
 *   max_loras           adapter slots, 1 <= max_loras <= LORA_MAX_LORAS.
 *   meta                host pointer to the output buffers (all non-null).
 *
 * Writes sorted_token_ids[0:num_tokens], all max_loras entries of the three
 * per-slot arrays, num_active, the padded tiles below num_tiles with
 * num_tiles, and num_runs.  A stable counting sort: bit-for-bit
 * deterministic, no atomics on global memory.  Grid: max_loras + 1
 * workgroups (of 64, 256, 512 or 1024 threads by max_tokens).
 */
lora_status_t lora_prepare_metadata(const int32_t *token_lora_mapping, int32_t num_tokens,
                                    int32_t max_tokens, int32_t max_loras,
                                    const lora_meta_t *meta, hipStream_t stream);

/*
 * lora_prepare_metadata_grouped - lora_prepare_metadata for a batch that
 * arrives grouped by adapter: every group (each adapter id, and the tokens
 * without an adapter) occupies one contiguous run of the batch, in any order
 * of the runs.
 *
 * Defined by: vLLM PR #13096, "Why do we need a new set of kernels" (the V0
 * path grouped the requests by LoRA id and its kernels relied on it) and the
 * MLC-LLM issue's Overview (Punica's segment vector, one segment per run).
 *
 * Arguments and outputs: exactly those of lora_prepare_metadata, bit for bit.
 * One workgroup reads the map once (O(num_tokens) work in all) and derives
 * every output from the run boundaries.  A batch that is NOT grouped is
 * detected on the device in the same launch and handled by the general
 * per-group code, group after group in that one workgroup: the same outputs,
 * at (max_loras + 1) passes over the map (use lora_prepare_metadata for such
 * batches).  Grid: one workgroup of 1024 threads.
 */
lora_status_t lora_prepare_metadata_grouped(const int32_t *token_lora_mapping,
                                            int32_t num_tokens, int32_t max_tokens,
                                            int32_t max_loras, const lora_meta_t *meta,
                                            hipStream_t stream);

/*
 * lora_shrink_default_splits - recommended number of hidden-dimension
 * partitions for lora_shrink (host only, no device access).  Returns a value in
 * [1, LORA_MAX_SPLITS], or 0 if an argument is out of range.  The result is a
 * pure function of its arguments: a rule on the sizes alone.  The best value
 * also depends on how the batch's tiles round against the compute units; the
 * Python helper segmented_rank_gemm_amd.tuning.tune_shrink_splits measures it
 * on a representative batch.
 */
int32_t lora_shrink_default_splits(int32_t hidden, int32_t max_tokens, int32_t max_loras,
                                   int32_t num_slices, int32_t rank);

/*
 * lora_shrink - gather each grouped token's activation row and project it onto
 * its adapter's A:  buf_p[s][t][k] = scale * sum_{h in part p} x[t][h] * A_s[l][k][h].
 *
 * Defined by: vLLM PR #13096 summary (the shrink kernel) and "Kernel Code
 * Change" item 2 (the input tokens are loaded through the token -> LoRA map);
 * the MLC-LLM issue's Overview (the per-segment low-rank multiplication).
 *
 *   x           bf16 [max_tokens][ldx]; columns [0, hidden) are read for the
 *               tokens that have an adapter.  Rows [0, max_tokens) must be
 *               addressable.  16-byte aligned.
 *   ldx         row stride of x in elements; ldx >= hidden, multiple of 8.
 *   hidden      input width; multiple of 8, 8 <= hidden <= 65536.
 *   lora_a      host array [num_slices] of device pointers, each
 *               bf16 [max_loras][rank][hidden], 16-byte aligned.
 *   num_slices  1 <= num_slices <= LORA_MAX_SLICES.
 *   rank        one of 8, 16, 32, 64 (LORA_ERR_UNSUPPORTED otherwise).
 *   scale       applied once, to every partial sum.
 *   buf         fp32 [num_splits][num_slices][max_tokens][rank], 16-byte
 *               aligned.  Part p holds the contribution of the p-th of
 *               num_splits contiguous ranges of the hidden dimension; the
 *               projection is the sum of the parts (with num_splits == 1 the
 *               buffer is the projection itself).  Only rows of tokens with an
 *               adapter are written, in every part.
 *   num_splits  1 <= num_splits <= LORA_MAX_SPLITS (see
 *               lora_shrink_default_splits); lora_expand must be given the
 *               same value.
 *   meta        output of lora_prepare_metadata for this batch.
 */
lora_status_t lora_shrink(const uint16_t *x, int64_t ldx, int32_t hidden,
                          const uint16_t *const *lora_a, int32_t num_slices, int32_t rank,
                          float scale, float *buf, int32_t num_splits, const lora_meta_t *meta,
                          int32_t max_tokens, int32_t max_loras, hipStream_t stream);

/*
 * lora_prepare_and_shrink - lora_prepare_metadata followed by lora_shrink for
 * the same batch, in one launch where the sizes allow it.
 *
 * Defined by: the two passages cited above (the grouping of an ungrouped
 * batch, vLLM PR #13096 "Why do we need a new set of kernels"; the shrink
 * kernel, its summary and "Kernel Code Change" item 2).  The fusion is this
 * library's: a V1 step computes the grouping and the first layer's shrink back
 * to back, and a launch boundary costs about as much as either kernel on a
 * small batch.
 *
 * Arguments: those of lora_prepare_metadata (token_lora_mapping, num_tokens,
 * max_tokens, max_loras, meta) and of lora_shrink (x, ldx, hidden, lora_a,
 * num_slices, rank, scale, buf, num_splits), with the same meanings and
 * checks.  Writes exactly what the two calls write, bit for bit (meta in
 * full, buf rows of tokens with an adapter).
 *
 * With max_tokens <= 512 one kernel is enqueued when max_loras * num_slices *
 * rank <= 256 (the shrink then takes tiles of 16 consecutive tokens in batch
 * order and the outputs of every adapter slot, each token keeping its own
 * adapter's) or max_loras <= 16 (the shrink finds each grouped tile's tokens
 * from the map itself); the last max_loras + 1 workgroups compute the
 * metadata.  Other sizes enqueue the metadata kernel and the shrink one after
 * the other.  The grid still depends only on the sizes, so the call can be
 * captured in a graph.
 */
lora_status_t lora_prepare_and_shrink(const int32_t *token_lora_mapping, int32_t num_tokens,
                                      const uint16_t *x, int64_t ldx, int32_t hidden,
                                      const uint16_t *const *lora_a, int32_t num_slices,
                                      int32_t rank, float scale, float *buf, int32_t num_splits,
                                      const lora_meta_t *meta, int32_t max_tokens,
                                      int32_t max_loras, hipStream_t stream);

/*
 * Launch choices of lora_expand (host struct; every field has a "the library's
 * rule" value).  They change how the work is cut and walked, never the result:
 * any valid setting gives the same bits.  A per-shape table of measured
 * choices is kept by the Python package (segmented_rank_gemm_amd.tuning).
 *   chunks_per_range   128-column chunks of a unit: per wave at ranks 8/16
 *                      (a unit spans 4x that), per workgroup at ranks 32/64.
 *                      0: rule; 1..64 (1..16 at ranks 32/64).
 *   range_fastest      unit order: 1 = a tile's column ranges one after
 *                      another, 0 = tiles one after another; -1: rule.
 *   workgroups_per_cu  workgroups per CU the persistent grid is sized for (no
 *                      more than the kernel holds at once); 0: rule; 1..16.
 */
typedef struct lora_expand_config {
  int32_t chunks_per_range;
  int32_t range_fastest;
  int32_t workgroups_per_cu;
} lora_expand_config_t;

/*
 * lora_expand - project each grouped token's rank-r vector up through its
 * adapter's B and add it into the output, slice by slice:
 *   y[t][off_s + n] = bf16( y[t][off_s + n] + sum_k buf[s][t][k] * B_s[l][n][k] ),
 * where buf[s][t][k] is the fp32 sum over the num_splits parts, the sum is
 * accumulated in fp32 and the result is rounded to bf16 (nearest, ties even).
 *
 * Defined by: vLLM PR #13096 summary (the expand kernel); the MLC-LLM issue's
 * Overview (per-segment low-rank multiplication); several output slices per
 * call cover fused projections such as qkv and gate_up.
 *
 *   buf         fp32 [num_splits][num_slices][max_tokens][rank], written by
 *               lora_shrink with the same num_splits.
 *   lora_b      host array [num_slices] of device pointers, each
 *               bf16 [max_loras][slice_sizes[s]][rank], 16-byte aligned.
 *   slice_sizes host array [num_slices]; each a multiple of 8, >= 8.
 *   y           bf16 [max_tokens][ldy], updated in place: only rows of tokens
 *               with an adapter, only columns [0, sum of slice_sizes).
 *               16-byte aligned.
 *   ldy         row stride of y in elements; >= sum of slice_sizes, multiple
 *               of 8.
 *   config      host pointer to launch choices, or NULL for the library's
 *               rules; an out-of-range field is LORA_ERR_INVALID_ARGUMENT.
 *   Other arguments as in lora_shrink.
 */
lora_status_t lora_expand(const float *buf, int32_t num_splits, const uint16_t *const *lora_b,
                          const int32_t *slice_sizes, int32_t num_slices, int32_t rank,
                          uint16_t *y, int64_t ldy, const lora_meta_t *meta, int32_t max_tokens,
                          int32_t max_loras, const lora_expand_config_t *config,
                          hipStream_t stream);

/*
 * lora_fused_step - the whole step for one batch (lora_prepare_metadata,
 * lora_shrink, lora_expand), in one launch where the sizes allow it.
 *
 * Defined by: the passages cited for the three calls (vLLM PR #13096, "Why do
 * we need a new set of kernels" and "Kernel Code Change" items 1 and 2; the
 * shrink and expand kernels of its summary) and the MLC-LLM issue's Overview:
 * Punica's single launch over every segment of the batch.
 *
 * Arguments: those of lora_prepare_metadata, lora_shrink and lora_expand for
 * the same batch (same meanings and checks), plus
 *   workspace        device memory of at least
 *                    lora_fused_step_workspace_bytes(...) bytes, 256-byte
 *                    aligned, ZERO-FILLED before its first use.  It holds
 *                    integer counters, which every call leaves zero-filled
 *                    again once it has completed, and, for the part sums
 *                    below, a scratch plane that each call overwrites before
 *                    reading it.  May be NULL when that size is 0.  Two calls
 *                    that overlap in time must not share a workspace (one
 *                    stream, or one workspace per stream).
 *   workspace_bytes  its size.
 *   options          host pointer, may be NULL (defaults).
 * Writes what the three calls write: meta in full, buf (num_splits parts) at
 * rows of tokens with an adapter, y at those rows and columns [0, sum n).
 *
 * One launch when max_tokens <= 512, rank is 8 or 16, max_loras * rank <= 64
 * and max_loras * num_slices * rank <= 256 (lora_fused_step_workspace_bytes
 * is then non-zero): tiles of 16 consecutive tokens in batch order; the
 * shrink's workgroups hand each tile's parts to the expand's through the
 * workspace's integer counters (bounded waits, no floating-point atomics; the
 * results are the same bits on every run).  Other sizes: lora_prepare_and_shrink
 * then lora_expand.  On that path, for max_tokens > 512 at rank 32 or 64 with
 * num_splits >= 2 (the workspace size is then non-zero), options->part_sums
 * = 1 has the shrink also hand the expand each row's rank vector summed over
 * the parts: the last shrink workgroup of each 64-token tile and output group
 * (integer arrival counters in the workspace) adds the parts in the order the
 * expand would, into the workspace's plane, and the expand reads that one
 * plane instead of every part (the same bits as without it; buf is written as
 * always).
 */
typedef struct lora_step_options {
  /* Upper bound on the polls of each cross-workgroup wait; a workgroup that
   * reaches it computes the missing parts itself (same bits, more time).
   * Negative: the default (65536).  0: never wait. */
  int32_t wait_polls;
  /* Launch choices of the expand on the multi-launch path (see lora_expand). */
  lora_expand_config_t expand;
  /* One-launch path: how long (ns) each expand workgroup holds its own B
   * loads back after it starts, so that the shrink workgroups' loads, which
   * share each CU's fetch path with them, are served first (its y loads: see
   * y_delay_ns).  Changes timing only, never results.  Negative: a default
   * from the shrink's per-workgroup bytes; 0: no hold-off; above 100000:
   * LORA_ERR_INVALID_ARGUMENT. */
  int32_t start_delay_ns;
  /* Multi-launch path, large batches at rank 32 or 64: 1 = the shrink sums
   * the parts for the expand (see above); 0 or negative = the expand sums
   * them (the default: the shrink's arrival round trips and the last
   * workgroup's read-back cost about what the expand saves). */
  int32_t part_sums;
  /* Multi-launch path, max_tokens > 512: 1 = the first launch is the shrink in
   * batch order (64-token tiles of consecutive tokens, each adapter present in
   * a tile one pass over its x rows) beside the metadata workgroups, instead
   * of the metadata kernel then the grouped shrink; the same bits.  Faster on
   * batches of request runs (a tile holds one or two adapters), slower on maps
   * drawn per token.  0 or negative: off (the default).  Ignored together
   * with part_sums = 1. */
  int32_t batch_order_shrink;
  /* One-launch path: the same for the expand workgroups' y loads, which go
   * out before their B loads (y comes from HBM, B mostly from L2); a value
   * above start_delay_ns issues B right after y.  Same range and meaning of
   * negative and 0. */
  int32_t y_delay_ns;
} lora_step_options_t;

int64_t lora_fused_step_workspace_bytes(int32_t max_tokens, int32_t max_loras,
                                        int32_t num_slices, int32_t rank);

/* lora_fused_step_launches - host-only query: 1 when lora_fused_step runs
 * the step in one launch for these sizes, 2 when it runs
 * lora_prepare_and_shrink then lora_expand, 0 for sizes it rejects. */
int32_t lora_fused_step_launches(int32_t max_tokens, int32_t max_loras, int32_t num_slices,
                                 int32_t rank);

lora_status_t lora_fused_step(const int32_t *token_lora_mapping, int32_t num_tokens,
                              const uint16_t *x, int64_t ldx, int32_t hidden,
                              const uint16_t *const *lora_a, const uint16_t *const *lora_b,
                              const int32_t *slice_sizes, int32_t num_slices, int32_t rank,
                              float scale, float *buf, int32_t num_splits, uint16_t *y,
                              int64_t ldy, const lora_meta_t *meta, void *workspace,
                              int64_t workspace_bytes, const lora_step_options_t *options,
                              int32_t max_tokens, int32_t max_loras, hipStream_t stream);

/*
 * lora_fused_step_static - lora_fused_step without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture
 * that must not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation).  Nothing is allocated: the one-launch path keeps its counters
 * in a file-scope device array of the library, 8 KB, enough for its largest
 * batch (512 token slots); each GPU the library runs on holds its own copy
 * until the process ends.  The array is zero-filled when the library's code
 * object is loaded and every call leaves it zero-filled again.  All calls on
 * one GPU share that GPU's array: calls that overlap in time on one GPU (two
 * streams, or two threads) race on it; order them on one stream.  The device
 * is the calling thread's current device (that of `stream`); the array's
 * device address is looked up on the first call on each device.
 *
 * Arguments, outputs, sizes and the multi-launch path for other sizes: as
 * lora_fused_step, except that options->part_sums is ignored (the part sums
 * need a workspace; the expand then sums the parts, the same bits).  A size whose counters would not fit the array returns
 * LORA_ERR_UNSUPPORTED with nothing enqueued (no size the one-launch path
 * accepts does); a failed lookup of the array returns LORA_ERR_LAUNCH.
 */
lora_status_t lora_fused_step_static(const int32_t *token_lora_mapping, int32_t num_tokens,
                                     const uint16_t *x, int64_t ldx, int32_t hidden,
                                     const uint16_t *const *lora_a,
                                     const uint16_t *const *lora_b, const int32_t *slice_sizes,
                                     int32_t num_slices, int32_t rank, float scale, float *buf,
                                     int32_t num_splits, uint16_t *y, int64_t ldy,
                                     const lora_meta_t *meta, const lora_step_options_t *options,
                                     int32_t max_tokens, int32_t max_loras, hipStream_t stream);

/* lora_status_string - static, human-readable name of a status code. */
const char *lora_status_string(lora_status_t status);

/* The measurement aids lora_stream_copy and lora_stream_update live in a
 * library of their own: lora_measure.h, liblora_measure.so. */

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
