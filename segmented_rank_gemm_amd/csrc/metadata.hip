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
// grid is max_loras + 1 workgroups whatever the ids are.  Every workgroup
// builds the full histogram in LDS (order-free counts), derives its group's
// start and its slot among the adapters present, then walks the map in token
// order and places its members with a ballot prefix count: position = start +
// number of earlier members.  No workgroup depends on another and no global
// atomic is used, so the result is the same bits on every run.

#include "device_common.hpp"

namespace lora {

constexpr int kMetaThreads = 1024;
constexpr int kMetaWaves = kMetaThreads / kWave;

__device__ __forceinline__ int group_of(int32_t id, int max_loras) {
  return (id >= -1 && id < max_loras) ? id + 1 : 0;
}

__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(
    const int32_t* __restrict__ mapping, int num_tokens, int max_loras,
    int32_t* __restrict__ sorted, int32_t* __restrict__ active_ids,
    int32_t* __restrict__ counts, int32_t* __restrict__ starts,
    int32_t* __restrict__ num_active) {
  __shared__ int hist[LORA_MAX_LORAS + 1];
  __shared__ int wave_total[kMetaWaves];
  __shared__ int s_start, s_slot, s_present;

  const int g = blockIdx.x;
  const int groups = max_loras + 1;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int i = tid; i < groups; i += kMetaThreads) hist[i] = 0;
  __syncthreads();
  for (int t = tid; t < num_tokens; t += kMetaThreads) atomicAdd(&hist[group_of(mapping[t], max_loras)], 1);
  __syncthreads();

  // Start of group g (tokens in lower groups), its slot among the adapters
  // present (present adapters with a lower id), and the number present.
  if (wave == 0) {
    int below = 0, slot = 0, present = 0;
    for (int base = 0; base < groups; base += kWave) {
      const int i = base + lane;
      const int h = i < groups ? hist[i] : 0;
      below += wave_sum(i < g ? h : 0);
      slot += __popcll(__ballot(i >= 1 && i < g && h > 0));
      present += __popcll(__ballot(i >= 1 && i < groups && h > 0));
    }
    if (lane == 0) {
      s_start = below;
      s_slot = slot;
      s_present = present;
    }
  }
  __syncthreads();

  const int members = hist[g];
  if (g == 0) {
    for (int i = s_present + tid; i < max_loras; i += kMetaThreads) {
      active_ids[i] = -1;
      counts[i] = 0;
      starts[i] = num_tokens;
    }
    if (tid == 0) *num_active = s_present;
  } else if (members > 0 && tid == 0) {
    active_ids[s_slot] = g - 1;
    counts[s_slot] = members;
    starts[s_slot] = s_start;
  }
  if (members == 0) return;  // uniform across the workgroup

  const unsigned long long below_lane = (1ull << lane) - 1ull;
  int base = s_start;
  for (int c = 0; c < num_tokens; c += kMetaThreads) {
    const int t = c + tid;
    const bool mine = t < num_tokens && group_of(mapping[t], max_loras) == g;
    const unsigned long long ballot = __ballot(mine);
    if (lane == 0) wave_total[wave] = __popcll(ballot);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kMetaWaves; ++w) {
      const int n = wave_total[w];
      before += w < wave ? n : 0;
      total += n;
    }
    const int pos = base + before + __popcll(ballot & below_lane);
    if (mine && pos < num_tokens) sorted[pos] = t;
    base += total;
    __syncthreads();
  }
}

hipError_t launch_metadata(const int32_t* mapping, int num_tokens, int max_loras,
                           const lora_meta_t& meta, hipStream_t stream) {
  hipLaunchKernelGGL(metadata_kernel, dim3(max_loras + 1), dim3(kMetaThreads), 0, stream,
                     mapping, num_tokens, max_loras, meta.sorted_token_ids, meta.active_lora_ids,
                     meta.num_tokens_per_lora, meta.lora_token_start, meta.num_active);
  return hipGetLastError();
}

}  // namespace lora
