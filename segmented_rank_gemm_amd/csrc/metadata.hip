// Metadata step: a stable counting sort of the batch's token indices by
// adapter id, on the device, with no host synchronisation.
//
// vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1" ("Why do we need a
// new set of kernels"): a V1 batch is not grouped by LoRA id, so the grouping
// the kernels rely on is built per batch from the token -> LoRA map.  vLLM PR
// #14626 "[Kernel] LoRA - Enable CUDAGraphs for V1": the buffers are static,
// sized by the maximum token count, so the launch must be too.
//
// One workgroup per group (group 0 = no adapter, group g = adapter g-1), so the
// grid is max_loras + 1 workgroups whatever the ids are.  The map is walked in
// blocks, kPerThread consecutive tokens per thread, each token read once (twice
// for batches larger than one block).  For its group g a workgroup needs three things: how many
// tokens sit in lower groups (its start), which groups occur at all (its slot
// among the adapters present and, for group 0, how many there are), and, per
// member, how many members precede it in token order (its rank).  Counts come
// from wave ballots summed in a fixed order, occurrence from an LDS flag
// per group, ranks from a block-wide exclusive scan of the per-thread member
// counts; no global atomics, so the result is the same bits on every run.
//
// The same workgroup also writes its adapter's run of the padded grouped order
// (16-token tiles of one adapter each, read by the kernels at fixed
// addresses): the run starts at round_up(S + 15 * k, 16), S being the tokens
// of lower adapters and k the group's slot, so it needs no other group's size.

#include "metadata_group.hpp"

namespace lora {

// THREADS threads per workgroup: the fewest whose block (THREADS * 8 tokens)
// holds the whole batch, up to 1024 (64, a single wave, up to 512 token slots;
// 256 up to 2048; 512 up to 4096; else 1024): the map is then read once and
// kept in registers, with the fewest waves to synchronise.  (Measured on a
// 4096-slot batch with 65 groups: 4.2 us at 512 threads, 5.1 us at 1024; on an
// 8192-slot batch two blocks of 512 threads cost 7.1 us against 5.7 us for one
// of 1024.)  Workgroup g owns group g.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void metadata_kernel(const int32_t* __restrict__ mapping,
                                                           int num_tokens, int max_loras,
                                                           MetaOut out) {
  metadata_group<THREADS>(mapping, num_tokens, max_loras, out, blockIdx.x);
}

hipError_t launch_metadata(const int32_t* mapping, int num_tokens, int max_tokens, int max_loras,
                           const lora_meta_t& meta, hipStream_t stream) {
  const MetaOut out{meta.sorted_token_ids, meta.active_lora_ids, meta.num_tokens_per_lora,
                    meta.lora_token_start, meta.num_active, meta.tile_token_ids,
                    meta.tile_lora, meta.num_tiles, meta.num_runs};
  if (max_tokens <= 64 * kPerThread) {
    hipLaunchKernelGGL(metadata_kernel<64>, dim3(max_loras + 1), dim3(64), 0, stream, mapping,
                       num_tokens, max_loras, out);
  } else if (max_tokens <= 256 * kPerThread) {
    hipLaunchKernelGGL(metadata_kernel<256>, dim3(max_loras + 1), dim3(256), 0, stream, mapping,
                       num_tokens, max_loras, out);
  } else if (max_tokens <= 512 * kPerThread) {
    hipLaunchKernelGGL(metadata_kernel<512>, dim3(max_loras + 1), dim3(512), 0, stream, mapping,
                       num_tokens, max_loras, out);
  } else {
    hipLaunchKernelGGL(metadata_kernel<1024>, dim3(max_loras + 1), dim3(1024), 0, stream, mapping,
                       num_tokens, max_loras, out);
  }
  return hipGetLastError();
}

}  // namespace lora
