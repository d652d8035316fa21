// C ABI of the multi-LoRA shrink/expand library: host-side argument checks,
// then exactly one kernel launch per call on the caller's stream.  No call
// allocates, synchronises or keeps state; launch grids depend only on the size
// arguments, so captured graphs stay valid for any batch of the same sizes
// (vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1", "Kernel Code
// Change" item 1; vLLM PR #14626 "[Kernel] LoRA - Enable CUDAGraphs for V1").

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_mi355x.h"

namespace lora {
hipError_t launch_metadata(const int32_t* mapping, int num_tokens, int max_tokens, int max_loras,
                           const lora_meta_t& meta, hipStream_t stream);
hipError_t launch_metadata_grouped(const int32_t* mapping, int num_tokens, int max_tokens,
                                   int max_loras, const lora_meta_t& meta, hipStream_t stream);
hipError_t launch_shrink(const uint16_t* x, int64_t ldx, int hidden, const uint16_t* const* lora_a,
                         int num_slices, int rank, float scale, float* buf, int num_splits,
                         const lora_meta_t& meta, int max_tokens, int max_loras, int num_cus,
                         hipStream_t stream, int* part_counters = nullptr,
                         float* part_sum = nullptr);
hipError_t launch_expand(const float* buf, int num_splits, const uint16_t* const* lora_b,
                         const int32_t* slice_sizes, int num_slices, int rank, uint16_t* y,
                         int64_t ldy, const lora_meta_t& meta, int max_tokens, int max_loras,
                         int num_cus, const lora_expand_config_t* config, hipStream_t stream,
                         const float* part_sum = nullptr);
int64_t part_sum_workspace_bytes(int max_tokens, int max_loras, int num_slices, int rank);
void part_sum_layout(void* workspace, int max_tokens, int max_loras, int num_slices, int rank,
                     int num_splits, int** counters, float** plane);
hipError_t launch_prep_shrink(const int32_t* mapping, int num_tokens, const uint16_t* x,
                              int64_t ldx, int hidden, const uint16_t* const* lora_a,
                              int num_slices, int rank, float scale, float* buf, int num_splits,
                              const lora_meta_t& meta, int max_tokens, int max_loras,
                              int num_cus, hipStream_t stream, int* part_counters = nullptr,
                              float* part_sum = nullptr, bool batch_order = false);
bool token_step_fits(int max_tokens, int max_loras, int num_slices, int rank);
int64_t token_step_workspace_bytes(int max_tokens);
hipError_t launch_token_step(const int32_t* mapping, int num_tokens, const uint16_t* x,
                             int64_t ldx, int hidden, const uint16_t* const* lora_a,
                             const uint16_t* const* lora_b, const int32_t* slice_sizes,
                             int num_slices, int rank, float scale, float* buf, int num_splits,
                             uint16_t* y, int64_t ldy, const lora_meta_t& meta, int* counters,
                             int wait_polls, int start_delay_ns, int y_delay_ns, int max_tokens,
                             int max_loras, hipStream_t stream);
int64_t token_step_scratch_bytes();
hipError_t token_step_scratch(int** out);
int shrink_group_blocks(int nb_total);
int shrink_tile_blocks(int max_tokens, int nb);
}  // namespace lora

namespace {

constexpr int32_t kMaxTokens = 1 << 24;
constexpr int32_t kMaxHidden = 65536;
constexpr int32_t kMaxStartDelayNs = 100000;  // lora_step_options_t.start_delay_ns, y_delay_ns

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool meta_ok(const lora_meta_t* m) {
  return m && m->sorted_token_ids && m->active_lora_ids && m->num_tokens_per_lora &&
         m->lora_token_start && m->num_active && m->tile_token_ids && m->tile_lora &&
         m->num_tiles && m->num_runs;
}

bool sizes_ok(int32_t max_tokens, int32_t max_loras) {
  return max_tokens >= 1 && max_tokens <= kMaxTokens && max_loras >= 1 &&
         max_loras <= LORA_MAX_LORAS;
}

bool rank_supported(int32_t rank) { return rank == 8 || rank == 16 || rank == 32 || rank == 64; }

// Compute units the persistent grids are sized for: the MI355X's 256 (a
// constant: no call queries the device for it).
int current_cus() { return 256; }

lora_status_t launch_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* lora_status_string(lora_status_t status) {
  switch (status) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARGUMENT: return "LORA_ERR_INVALID_ARGUMENT";
    case LORA_ERR_UNSUPPORTED: return "LORA_ERR_UNSUPPORTED";
    case LORA_ERR_LAUNCH: return "LORA_ERR_LAUNCH";
  }
  return "LORA_ERR_UNKNOWN";
}

lora_status_t lora_prepare_metadata(const int32_t* token_lora_mapping, int32_t num_tokens,
                                    int32_t max_tokens, int32_t max_loras,
                                    const lora_meta_t* meta, hipStream_t stream) {
  if (!meta_ok(meta) || !sizes_ok(max_tokens, max_loras)) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && !token_lora_mapping) return LORA_ERR_INVALID_ARGUMENT;
  return launch_status(
      lora::launch_metadata(token_lora_mapping, num_tokens, max_tokens, max_loras, *meta, stream));
}

lora_status_t lora_prepare_metadata_grouped(const int32_t* token_lora_mapping,
                                            int32_t num_tokens, int32_t max_tokens,
                                            int32_t max_loras, const lora_meta_t* meta,
                                            hipStream_t stream) {
  if (!meta_ok(meta) || !sizes_ok(max_tokens, max_loras)) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && !token_lora_mapping) return LORA_ERR_INVALID_ARGUMENT;
  return launch_status(lora::launch_metadata_grouped(token_lora_mapping, num_tokens, max_tokens,
                                                     max_loras, *meta, stream));
}

int32_t lora_shrink_default_splits(int32_t hidden, int32_t max_tokens, int32_t max_loras,
                                   int32_t num_slices, int32_t rank) {
  if (hidden < 8 || hidden > kMaxHidden || !sizes_ok(max_tokens, max_loras) || num_slices < 1 ||
      num_slices > LORA_MAX_SLICES || rank < 1 || rank > 64)
    return 0;
  // Enough (tile, part, output group) units for ~1 workgroup per CU of a
  // 256-CU device at the largest batch, with parts of at least 256 hidden
  // elements.  Small batches (16-token tiles) at ranks 8 and 16: parts of at
  // most 256 elements, one 64-element chunk per wave, the batch-order
  // shrink's fast path (measured through lora_fused_step, µs: qkv 3 x 4096,
  // rank 8, 512 tokens 22.3 at the former 15 parts -> 13.9 at 16; rank 16,
  // 256 tokens 18.4 at 8 -> 14.1 at 16; hidden 8192, rank 8, 256 tokens 15.6
  // at 16 -> 12.7 at 32; the two-call path gained too).  Other small batches:
  // ~2 units per CU, but no more parts than the expand sums with one batch of
  // loads (8) and parts * rank <= 256 (at most 1 KB of parts per token).
  // Large batches (64-token tiles): also parts of about 1400 elements (at
  // least 4), so that several workgroups share each CU, up to 8 parts
  // (measured on the prefill, down_proj and 70B shapes; a second batch of
  // loads in the expand at rank 64 costs far less than the shrink gains).
  const int nb_total = (num_slices * rank + 15) / 16;
  const int nb = lora::shrink_group_blocks(nb_total);
  const int64_t groups = (nb_total + nb - 1) / nb;
  const int mw = lora::shrink_tile_blocks(max_tokens, nb);
  const int64_t tile = 16 * mw;
  const int64_t tiles = (static_cast<int64_t>(max_tokens) + tile - 1) / tile + max_loras;
  int64_t splits = (256 + tiles * groups - 1) / (tiles * groups);
  const int64_t by_len = hidden / 256 > 0 ? hidden / 256 : 1;
  int64_t cap;
  if (mw != 4) splits = (512 + tiles * groups - 1) / (tiles * groups);
  if (mw == 4) {
    int64_t by_work = (hidden + 700) / 1400;  // parts of about 1400 elements, 4 to 8
    by_work = by_work < 4 ? 4 : by_work;
    splits = splits > by_work ? splits : by_work;
    // at rank 64 the expand sums up to six parts in one batch of loads
    // (down_proj, hidden 11008: 8 parts 47.2 us per step, 6 parts 43.6)
    cap = rank == 64 ? 6 : 8;
  } else if (rank <= 16) {
    splits = (hidden + 255) / 256;  // parts of at most 256 elements
    cap = LORA_MAX_SPLITS;
  } else {
    const int64_t group = 8;  // parts the expand sums per batch of loads
    cap = 256 / rank < group ? 256 / rank : group;
  }
  if (mw == 4 || rank > 16) splits = splits < by_len ? splits : by_len;
  splits = splits < cap ? splits : cap;
  splits = splits < 1 ? 1 : (splits > LORA_MAX_SPLITS ? LORA_MAX_SPLITS : splits);
  return static_cast<int32_t>(splits);
}

// Checks of lora_shrink's arguments (meta and sizes included).
static lora_status_t shrink_args(const uint16_t* x, int64_t ldx, int32_t hidden,
                          const uint16_t* const* lora_a, int32_t num_slices, int32_t rank,
                          const float* buf, int32_t num_splits, const lora_meta_t* meta,
                          int32_t max_tokens, int32_t max_loras) {
  if (!meta_ok(meta) || !sizes_ok(max_tokens, max_loras)) return LORA_ERR_INVALID_ARGUMENT;
  if (!x || !lora_a || !buf || !aligned16(x) || !aligned16(buf)) return LORA_ERR_INVALID_ARGUMENT;
  if (hidden < 8 || hidden > kMaxHidden || hidden % 8 != 0) return LORA_ERR_INVALID_ARGUMENT;
  if (ldx < hidden || ldx % 8 != 0) return LORA_ERR_INVALID_ARGUMENT;
  if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_INVALID_ARGUMENT;
  if (num_splits < 1 || num_splits > LORA_MAX_SPLITS) return LORA_ERR_INVALID_ARGUMENT;
  if (rank < 1 || rank > 64) return LORA_ERR_INVALID_ARGUMENT;
  for (int32_t s = 0; s < num_slices; ++s)
    if (!lora_a[s] || !aligned16(lora_a[s])) return LORA_ERR_INVALID_ARGUMENT;
  if (!rank_supported(rank)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

lora_status_t lora_shrink(const uint16_t* x, int64_t ldx, int32_t hidden,
                          const uint16_t* const* lora_a, int32_t num_slices, int32_t rank,
                          float scale, float* buf, int32_t num_splits, const lora_meta_t* meta,
                          int32_t max_tokens, int32_t max_loras, hipStream_t stream) {
  const lora_status_t st = shrink_args(x, ldx, hidden, lora_a, num_slices, rank, buf, num_splits,
                                       meta, max_tokens, max_loras);
  if (st != LORA_OK) return st;
  return launch_status(lora::launch_shrink(x, ldx, hidden, lora_a, num_slices, rank, scale, buf,
                                           num_splits, *meta, max_tokens, max_loras,
                                           current_cus(), stream));
}

lora_status_t lora_prepare_and_shrink(const int32_t* token_lora_mapping, int32_t num_tokens,
                                      const uint16_t* x, int64_t ldx, int32_t hidden,
                                      const uint16_t* const* lora_a, int32_t num_slices,
                                      int32_t rank, float scale, float* buf, int32_t num_splits,
                                      const lora_meta_t* meta, int32_t max_tokens,
                                      int32_t max_loras, hipStream_t stream) {
  if (!meta_ok(meta) || !sizes_ok(max_tokens, max_loras)) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && !token_lora_mapping) return LORA_ERR_INVALID_ARGUMENT;
  const lora_status_t st = shrink_args(x, ldx, hidden, lora_a, num_slices, rank, buf, num_splits,
                                       meta, max_tokens, max_loras);
  if (st != LORA_OK) return st;
  return launch_status(lora::launch_prep_shrink(token_lora_mapping, num_tokens, x, ldx, hidden,
                                                lora_a, num_slices, rank, scale, buf, num_splits,
                                                *meta, max_tokens, max_loras, current_cus(),
                                                stream));
}

static bool expand_config_ok(const lora_expand_config_t* c, int32_t rank) {
  if (!c) return true;
  const int32_t max_cpr = rank >= 32 ? 16 : 64;
  return c->chunks_per_range >= 0 && c->chunks_per_range <= max_cpr && c->range_fastest >= -1 &&
         c->range_fastest <= 1 && c->workgroups_per_cu >= 0 && c->workgroups_per_cu <= 16;
}

lora_status_t lora_expand(const float* buf, int32_t num_splits, const uint16_t* const* lora_b,
                          const int32_t* slice_sizes, int32_t num_slices, int32_t rank,
                          uint16_t* y, int64_t ldy, const lora_meta_t* meta, int32_t max_tokens,
                          int32_t max_loras, const lora_expand_config_t* config,
                          hipStream_t stream) {
  if (!meta_ok(meta) || !sizes_ok(max_tokens, max_loras)) return LORA_ERR_INVALID_ARGUMENT;
  if (!buf || !lora_b || !slice_sizes || !y || !aligned16(buf) || !aligned16(y))
    return LORA_ERR_INVALID_ARGUMENT;
  if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_INVALID_ARGUMENT;
  if (num_splits < 1 || num_splits > LORA_MAX_SPLITS) return LORA_ERR_INVALID_ARGUMENT;
  if (rank < 1 || rank > 64) return LORA_ERR_INVALID_ARGUMENT;
  int64_t n_total = 0;
  for (int32_t s = 0; s < num_slices; ++s) {
    if (!lora_b[s] || !aligned16(lora_b[s])) return LORA_ERR_INVALID_ARGUMENT;
    if (slice_sizes[s] < 8 || slice_sizes[s] % 8 != 0) return LORA_ERR_INVALID_ARGUMENT;
    n_total += slice_sizes[s];
  }
  if (n_total > (int64_t{1} << 30) || ldy < n_total || ldy % 8 != 0) return LORA_ERR_INVALID_ARGUMENT;
  if (!expand_config_ok(config, rank)) return LORA_ERR_INVALID_ARGUMENT;
  if (!rank_supported(rank)) return LORA_ERR_UNSUPPORTED;
  return launch_status(lora::launch_expand(buf, num_splits, lora_b, slice_sizes, num_slices, rank,
                                           y, ldy, *meta, max_tokens, max_loras, current_cus(),
                                           config, stream));
}

int64_t lora_fused_step_workspace_bytes(int32_t max_tokens, int32_t max_loras,
                                        int32_t num_slices, int32_t rank) {
  if (!sizes_ok(max_tokens, max_loras) || num_slices < 1 || num_slices > LORA_MAX_SLICES)
    return 0;
  if (lora::token_step_fits(max_tokens, max_loras, num_slices, rank))
    return lora::token_step_workspace_bytes(max_tokens);
  return lora::part_sum_workspace_bytes(max_tokens, max_loras, num_slices, rank);
}

int32_t lora_fused_step_launches(int32_t max_tokens, int32_t max_loras, int32_t num_slices,
                                 int32_t rank) {
  if (!sizes_ok(max_tokens, max_loras) || num_slices < 1 || num_slices > LORA_MAX_SLICES ||
      !(rank == 8 || rank == 16 || rank == 32 || rank == 64))
    return 0;
  return lora::token_step_fits(max_tokens, max_loras, num_slices, rank) ? 1 : 2;
}

// Checks of lora_expand's arguments other than meta and the sizes.
static lora_status_t expand_args(const float* buf, int32_t num_splits,
                                 const uint16_t* const* lora_b, const int32_t* slice_sizes,
                                 int32_t num_slices, int32_t rank, const uint16_t* y, int64_t ldy) {
  if (!buf || !lora_b || !slice_sizes || !y || !aligned16(buf) || !aligned16(y))
    return LORA_ERR_INVALID_ARGUMENT;
  if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_INVALID_ARGUMENT;
  if (num_splits < 1 || num_splits > LORA_MAX_SPLITS) return LORA_ERR_INVALID_ARGUMENT;
  if (rank < 1 || rank > 64) return LORA_ERR_INVALID_ARGUMENT;
  int64_t n_total = 0;
  for (int32_t s = 0; s < num_slices; ++s) {
    if (!lora_b[s] || !aligned16(lora_b[s])) return LORA_ERR_INVALID_ARGUMENT;
    if (slice_sizes[s] < 8 || slice_sizes[s] % 8 != 0) return LORA_ERR_INVALID_ARGUMENT;
    n_total += slice_sizes[s];
  }
  if (n_total > (int64_t{1} << 30) || ldy < n_total || ldy % 8 != 0)
    return LORA_ERR_INVALID_ARGUMENT;
  if (!rank_supported(rank)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

static const lora_expand_config_t* options_expand(const lora_step_options_t* options) {
  return options ? &options->expand : nullptr;
}

// lora_fused_step and lora_fused_step_static: argument checks, then the
// one-launch kernel on `counters` (from the caller's workspace or the
// library's static array, resolved only once the arguments are known to be
// valid and the one-launch path is taken) or the multi-launch path.
// static_counters: use the library's array instead of workspace.
static lora_status_t fused_step(const int32_t* token_lora_mapping, int32_t num_tokens,
                                const uint16_t* x, int64_t ldx, int32_t hidden,
                                const uint16_t* const* lora_a, const uint16_t* const* lora_b,
                                const int32_t* slice_sizes, int32_t num_slices, int32_t rank,
                                float scale, float* buf, int32_t num_splits, uint16_t* y,
                                int64_t ldy, const lora_meta_t* meta, void* workspace,
                                int64_t workspace_bytes, bool static_counters,
                                const lora_step_options_t* options, int32_t max_tokens,
                                int32_t max_loras, hipStream_t stream) {
  if (!meta_ok(meta) || !sizes_ok(max_tokens, max_loras)) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens) return LORA_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && !token_lora_mapping) return LORA_ERR_INVALID_ARGUMENT;
  lora_status_t st = shrink_args(x, ldx, hidden, lora_a, num_slices, rank, buf, num_splits, meta,
                                 max_tokens, max_loras);
  if (st != LORA_OK) return st;
  st = expand_args(buf, num_splits, lora_b, slice_sizes, num_slices, rank, y, ldy);
  if (st != LORA_OK) return st;
  if (!expand_config_ok(options_expand(options), rank)) return LORA_ERR_INVALID_ARGUMENT;
  if (options && (options->start_delay_ns > kMaxStartDelayNs ||
                  options->y_delay_ns > kMaxStartDelayNs))
    return LORA_ERR_INVALID_ARGUMENT;
  const int64_t need = lora_fused_step_workspace_bytes(max_tokens, max_loras, num_slices, rank);
  const bool one_launch = lora::token_step_fits(max_tokens, max_loras, num_slices, rank);
  if (need > 0 && one_launch) {
    int* counters = nullptr;
    if (static_counters) {
      if (need > lora::token_step_scratch_bytes()) return LORA_ERR_UNSUPPORTED;
      if (lora::token_step_scratch(&counters) != hipSuccess) return LORA_ERR_LAUNCH;
    } else {
      if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
          workspace_bytes < need)
        return LORA_ERR_INVALID_ARGUMENT;
      counters = static_cast<int*>(workspace);
    }
    const int polls = options && options->wait_polls >= 0 ? options->wait_polls : 65536;
    const int delay = options ? options->start_delay_ns : -1;
    const int y_delay = options ? options->y_delay_ns : -1;
    return launch_status(lora::launch_token_step(
        token_lora_mapping, num_tokens, x, ldx, hidden, lora_a, lora_b, slice_sizes, num_slices,
        rank, scale, buf, num_splits, y, ldy, *meta, counters, polls, delay, y_delay, max_tokens,
        max_loras, stream));
  }
  // Multi-launch path.  With a workspace (large batches at ranks 32 and 64):
  // the shrink also hands the expand its parts summed per row.
  int* part_counters = nullptr;
  float* part_sum = nullptr;
  if (need > 0 && !static_counters && options && options->part_sums > 0) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_bytes < need)
      return LORA_ERR_INVALID_ARGUMENT;
    lora::part_sum_layout(workspace, max_tokens, max_loras, num_slices, rank, num_splits,
                          &part_counters, &part_sum);
  }
  st = launch_status(lora::launch_prep_shrink(token_lora_mapping, num_tokens, x, ldx, hidden,
                                              lora_a, num_slices, rank, scale, buf, num_splits,
                                              *meta, max_tokens, max_loras, current_cus(), stream,
                                              part_counters, part_sum,
                                              options && options->batch_order_shrink > 0 &&
                                                  part_sum == nullptr));
  if (st != LORA_OK) return st;
  return launch_status(lora::launch_expand(buf, num_splits, lora_b, slice_sizes, num_slices, rank,
                                           y, ldy, *meta, max_tokens, max_loras, current_cus(),
                                           options_expand(options), stream, part_sum));
}

lora_status_t lora_fused_step(const int32_t* token_lora_mapping, int32_t num_tokens,
                              const uint16_t* x, int64_t ldx, int32_t hidden,
                              const uint16_t* const* lora_a, const uint16_t* const* lora_b,
                              const int32_t* slice_sizes, int32_t num_slices, int32_t rank,
                              float scale, float* buf, int32_t num_splits, uint16_t* y,
                              int64_t ldy, const lora_meta_t* meta, void* workspace,
                              int64_t workspace_bytes, const lora_step_options_t* options,
                              int32_t max_tokens, int32_t max_loras, hipStream_t stream) {
  return fused_step(token_lora_mapping, num_tokens, x, ldx, hidden, lora_a, lora_b, slice_sizes,
                    num_slices, rank, scale, buf, num_splits, y, ldy, meta, workspace,
                    workspace_bytes, false, options, max_tokens, max_loras, stream);
}

lora_status_t lora_fused_step_static(const int32_t* token_lora_mapping, int32_t num_tokens,
                                     const uint16_t* x, int64_t ldx, int32_t hidden,
                                     const uint16_t* const* lora_a, const uint16_t* const* lora_b,
                                     const int32_t* slice_sizes, int32_t num_slices, int32_t rank,
                                     float scale, float* buf, int32_t num_splits, uint16_t* y,
                                     int64_t ldy, const lora_meta_t* meta,
                                     const lora_step_options_t* options, int32_t max_tokens,
                                     int32_t max_loras, hipStream_t stream) {
  return fused_step(token_lora_mapping, num_tokens, x, ldx, hidden, lora_a, lora_b, slice_sizes,
                    num_slices, rank, scale, buf, num_splits, y, ldy, meta, nullptr, 0, true,
                    options, max_tokens, max_loras, stream);
}

}  // extern "C"
