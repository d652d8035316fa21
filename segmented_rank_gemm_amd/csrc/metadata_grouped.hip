// Metadata step for a batch that arrives already grouped by adapter (every
// group's tokens contiguous in batch order): the V0 situation.
//
// vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1", "Why do we need a
// new set of kernels": the V0 path sorted / grouped the requests by LoRA id,
// which the SGMV kernels relied on; V1 does not.  MLC-LLM issue "[Tracking]
// Multi-LoRA Serving", Overview: Punica's segment vector, one entry per
// request run.  For such a batch the stable grouping is the identity inside
// each run, so the metadata follows from the run boundaries alone: one pass
// over the map, O(T) work in all (the general kernel has max_loras + 1
// workgroups each read the whole map).
//
// One workgroup (64, 256, 512 or 1024 threads: the fewest whose 8-token-per-
// thread block holds the batch, as for the metadata kernel):
//  1. blocks of 8 tokens per thread (in registers): a run starts where a
//     token's group (0: no adapter, id + 1 otherwise; ids outside
//     [-1, max_loras) count as no adapter) differs from the previous token's;
//     run starts are numbered in batch order by a block-wide scan of per-thread
//     counts (ballots) and recorded in LDS.  More runs than groups: not grouped.
//  2. a group with two runs: not grouped (LDS counters per group).
//  3. grouped: each group's count and first position from its run; exclusive
//     scans over the groups (ascending id, no adapter first) give the starts,
//     the adapter slots and the padded-tile starts (the metadata kernel's
//     round_up(S_k + 15 k, 16)); each thread then writes 8 consecutive output
//     positions (one binary search over the group starts, then a walk):
//     contiguous stores, no scatter.
//  4. not grouped: the general per-group code (metadata_group.hpp) for every
//     group in turn, in this workgroup: the same bits as lora_prepare_metadata,
//     at (max_loras + 1) passes over the map.
// Outputs are those of lora_prepare_metadata, bit for bit, either way.

#include "metadata_group.hpp"

namespace lora {

constexpr int kMaxGroups = LORA_MAX_LORAS + 1;

// Block-wide exclusive sum of v >= 0 over the workgroup's threads (thread
// order); also the total.  Uses `wsum` (one int of LDS per wave).  A
// one-wave workgroup needs no barrier.
template <int THREADS>
__device__ __forceinline__ int block_exclusive_sum(int v, int* wsum, int& total) {
  constexpr int kWaves = THREADS / kWave;
  const int ex = wave_exclusive_sum(v);
  if constexpr (kWaves == 1) {
    total = __builtin_amdgcn_readlane(ex + v, kWave - 1);
    return ex;
  }
  const int lane = lane_id();
  const int wave = wave_index();
  if (lane == kWave - 1) wsum[wave] = ex + v;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int n = wsum[w];
    before += w < wave ? n : 0;
    total += n;
  }
  __syncthreads();  // wsum is reused
  return before + ex;
}

// Last index i in [0, n) with a[i] <= key (a non-decreasing, a[0] <= key).
__device__ __forceinline__ int last_le(const int* a, int n, int key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= key) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Positions [p0, p0 + 8) of an int32 output below n: two 16-byte stores when
// all 8 are in range and aligned, else one store per position.
__device__ __forceinline__ void store_positions(int32_t* dst, int p0, int n,
                                                const int (&v)[kPerThread]) {
  if (p0 + kPerThread <= n && (reinterpret_cast<uintptr_t>(dst + p0) & 15) == 0) {
    store16(dst + p0, u32x4{static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]),
                            static_cast<uint32_t>(v[2]), static_cast<uint32_t>(v[3])});
    store16(dst + p0 + 4, u32x4{static_cast<uint32_t>(v[4]), static_cast<uint32_t>(v[5]),
                                static_cast<uint32_t>(v[6]), static_cast<uint32_t>(v[7])});
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (p0 + e < n) dst[p0 + e] = v[e];
  }
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void metadata_grouped_kernel(
    const int32_t* __restrict__ mapping, int num_tokens, int max_loras, MetaOut out) {
  constexpr int kBlock = THREADS * kPerThread;
  __shared__ int run_pos[kMaxGroups + 1];
  __shared__ int run_grp[kMaxGroups];
  __shared__ int g_cnt[kMaxGroups];    // tokens per group
  __shared__ int g_pos[kMaxGroups];    // first batch position of the group's run
  __shared__ int g_start[kMaxGroups];  // start in the grouped order
  __shared__ int g_runs[kMaxGroups];   // runs per group
  __shared__ int k_pstart[kMaxGroups];  // per adapter slot: padded start, count, first position
  __shared__ int k_cnt[kMaxGroups];
  __shared__ int k_pos[kMaxGroups];
  __shared__ int k_id[kMaxGroups];
  __shared__ int wsum[THREADS / kWave];
  __shared__ int s_runs, s_bad;

  const int tid = threadIdx.x;
  const int groups = max_loras + 1;
  for (int g = tid; g < groups; g += THREADS) {
    g_cnt[g] = 0;
    g_runs[g] = 0;
  }
  if (tid == 0) {
    s_runs = 0;
    s_bad = 0;
  }
  __syncthreads();

  // 1. run starts, numbered in batch order
  for (int b0 = 0; b0 < num_tokens; b0 += kBlock) {
    const int t0 = b0 + tid * kPerThread;
    int grp[kPerThread];
    load_groups(mapping, num_tokens, max_loras, t0, grp);
    int prev = -1;  // group of token t0 - 1; -1 before the first token
    if (t0 > 0 && t0 < num_tokens) prev = group_of(mapping[t0 - 1], max_loras);
    unsigned starts = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (grp[e] >= 0 && grp[e] != prev) starts |= 1u << e;
      prev = grp[e];
    }
    int total = 0;
    const int mine = __builtin_popcount(starts);
    const int ex = block_exclusive_sum<THREADS>(mine, wsum, total);
    const int base = s_runs;  // (read before the update below, after the scan's barriers)
    if (base + total > groups) {
      if (tid == 0) s_bad = 1;  // more runs than groups: some group has two
    } else {
      int r = base + ex;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        if (starts & (1u << e)) {
          run_pos[r] = t0 + e;
          run_grp[r] = grp[e];
          ++r;
        }
      }
    }
    __syncthreads();
    if (tid == 0) s_runs = base + total;
    __syncthreads();
    if (s_bad) break;  // workgroup-uniform
  }

  // 2. one run per group
  const int runs = s_runs;
  if (!s_bad) {
    if (tid == 0) run_pos[runs] = num_tokens;
    for (int r = tid; r < runs; r += THREADS)
      if (atomicAdd(&g_runs[run_grp[r]], 1) > 0) s_bad = 1;  // benign: every writer stores 1
    __syncthreads();
  }
  if (s_bad) {
    // 4. not grouped: the general code, group by group
    for (int g = 0; g < groups; ++g) metadata_group<THREADS>(mapping, num_tokens, max_loras, out, g);
    return;
  }

  // 3. grouped
  for (int r = tid; r < runs; r += THREADS) {
    const int g = run_grp[r];
    g_cnt[g] = run_pos[r + 1] - run_pos[r];
    g_pos[g] = run_pos[r];
  }
  __syncthreads();
  // starts (all groups) and slots (groups of adapters present): each thread
  // takes a contiguous range of groups, sums it, and the ranges' sums are
  // scanned across the workgroup
  constexpr int kMaxPer = (kMaxGroups + THREADS - 1) / THREADS;
  const int per = (groups + THREADS - 1) / THREADS;
  const int g0 = tid * per;
  int tok_sum = 0, pres_sum = 0;
  for (int i = 0; i < per; ++i) {
    const int g = g0 + i;
    if (g < groups) {
      tok_sum += g_cnt[g];
      pres_sum += (g >= 1 && g_cnt[g] > 0) ? 1 : 0;
    }
  }
  int ngroups_tokens = 0, npresent = 0;
  int start = block_exclusive_sum<THREADS>(tok_sum, wsum, ngroups_tokens);
  int slot = block_exclusive_sum<THREADS>(pres_sum, wsum, npresent);
  const int n_none = g_cnt[0];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int g = g0 + i;
    if (i < per && g < groups) {
      const int gc = g_cnt[g];
      g_start[g] = start;
      if (g >= 1 && gc > 0) {
        k_pstart[slot] = round_up_tile(start - n_none + (kMetaTile - 1) * slot);
        k_cnt[slot] = gc;
        k_pos[slot] = g_pos[g];
        k_id[slot] = g - 1;
        out.active_ids[slot] = g - 1;
        out.counts[slot] = gc;
        out.starts[slot] = start;
        ++slot;
      }
      start += gc;
    }
  }
  for (int i = npresent + tid; i < max_loras; i += THREADS) {
    out.active_ids[i] = -1;
    out.counts[i] = 0;
    out.starts[i] = num_tokens;
  }
  __syncthreads();
  const int num_tiles =
      npresent > 0 ? round_up_tile(k_pstart[npresent - 1] + k_cnt[npresent - 1]) / kMetaTile : 0;
  if (tid == 0) {
    *out.num_active = npresent;
    *out.num_runs = npresent;  // one run per adapter present
    *out.num_tiles = num_tiles;
  }

  // Outputs, 8 consecutive positions per thread: one binary search for the
  // first (the last group whose start is <= p: an empty group shares its start
  // with the next non-empty group, which comes later), then a walk forward;
  // 16-byte stores where the 8 positions are whole and aligned.
  for (int p0 = kPerThread * tid; p0 < num_tokens; p0 += kBlock) {
    int g = last_le(g_start, groups, p0);
    int v[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int p = p0 + e;
      while (g + 1 < groups && p >= g_start[g] + g_cnt[g]) ++g;
      v[e] = g_pos[g] + (p - g_start[g]);
    }
    store_positions(out.sorted, p0, num_tokens, v);
  }
  // the padded tiles: position q lies in the run of the last slot whose
  // padded start is <= q, or in the gap after it
  if (npresent > 0) {
    const int nq = num_tiles * kMetaTile;
    for (int q0 = kPerThread * tid; q0 < nq; q0 += kBlock) {
      int k = last_le(k_pstart, npresent, q0);
      int v[kPerThread];
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const int q = q0 + e;
        while (k + 1 < npresent && q >= k_pstart[k + 1]) ++k;
        const int j = q - k_pstart[k];
        v[e] = j < k_cnt[k] ? k_pos[k] + j : -1;
      }
      store_positions(out.tile_ids, q0, nq, v);
    }
    for (int m = tid; m < num_tiles; m += THREADS) {
      const int k = last_le(k_pstart, npresent, kMetaTile * m);
      out.tile_lora[m] = kMetaTile * m - k_pstart[k] < k_cnt[k] ? k_id[k] : -1;
    }
  }
}

hipError_t launch_metadata_grouped(const int32_t* mapping, int num_tokens, int max_tokens,
                                   int max_loras, const lora_meta_t& meta, hipStream_t stream) {
  const MetaOut out{meta.sorted_token_ids, meta.active_lora_ids, meta.num_tokens_per_lora,
                    meta.lora_token_start, meta.num_active, meta.tile_token_ids,
                    meta.tile_lora, meta.num_tiles, meta.num_runs};
  if (max_tokens <= 64 * kPerThread) {
    hipLaunchKernelGGL(metadata_grouped_kernel<64>, dim3(1), dim3(64), 0, stream, mapping,
                       num_tokens, max_loras, out);
  } else if (max_tokens <= 256 * kPerThread) {
    hipLaunchKernelGGL(metadata_grouped_kernel<256>, dim3(1), dim3(256), 0, stream, mapping,
                       num_tokens, max_loras, out);
  } else if (max_tokens <= 512 * kPerThread) {
    hipLaunchKernelGGL(metadata_grouped_kernel<512>, dim3(1), dim3(512), 0, stream, mapping,
                       num_tokens, max_loras, out);
  } else {
    hipLaunchKernelGGL(metadata_grouped_kernel<1024>, dim3(1), dim3(1024), 0, stream, mapping,
                       num_tokens, max_loras, out);
  }
  return hipGetLastError();
}

}  // namespace lora
