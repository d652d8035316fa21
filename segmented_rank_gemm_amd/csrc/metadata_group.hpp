// The metadata step's per-group work, shared by the metadata kernel and the
// fused prepare + shrink kernel: a workgroup of THREADS threads builds group g's
// part of the grouping (g = 0: tokens without an adapter, g = l + 1: adapter l).
// See metadata.hip for the method.
#pragma once

#include "device_common.hpp"

namespace lora {


constexpr int kPerThread = 8;

__device__ __forceinline__ int group_of(int32_t id, int max_loras) {
  return (id >= -1 && id < max_loras) ? id + 1 : 0;
}

// Groups of this thread's kPerThread consecutive tokens starting at t0 (-1 past
// the end of the batch).
__device__ __forceinline__ void load_groups(const int32_t* __restrict__ mapping, int num_tokens,
                                            int max_loras, int t0, int (&grp)[kPerThread]) {
  if (t0 + kPerThread <= num_tokens && (reinterpret_cast<uintptr_t>(mapping + t0) & 15) == 0) {
    const u32x4 a = load16(mapping + t0);
    const u32x4 c = load16(mapping + t0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      grp[e] = group_of(static_cast<int32_t>(a[e]), max_loras);
      grp[4 + e] = group_of(static_cast<int32_t>(c[e]), max_loras);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      grp[e] = t0 + e < num_tokens ? group_of(mapping[t0 + e], max_loras) : -1;
  }
}

struct MetaOut {
  int32_t* sorted;
  int32_t* active_ids;
  int32_t* counts;
  int32_t* starts;
  int32_t* num_active;
  int32_t* tile_ids;
  int32_t* tile_lora;
  int32_t* num_tiles;
  int32_t* num_runs;
};

constexpr int kMetaTile = LORA_TILE;

__device__ __forceinline__ int round_up_tile(int v) {
  return (v + kMetaTile - 1) / kMetaTile * kMetaTile;
}

// LDS of one metadata workgroup.
template <int THREADS>
struct MetaLds {
  static constexpr int kWaves = THREADS / kWave;
  int present[LORA_MAX_LORAS + 1];
  int wave_below[kWaves], wave_members[kWaves], wave_none[kWaves], wave_scan[kWaves];
  int wave_runs[kWaves];
  int32_t staged[THREADS * kPerThread];  // one block's members of g, in rank order
};

// Group g's share of the metadata, by one workgroup of THREADS threads (every
// thread of the workgroup calls it); a block of the map is THREADS * 8 tokens.
// `sh`: the workgroup's LDS for it (a kernel whose other workgroups need more
// LDS for other work passes part of that, so that it does not add to it).
template <int THREADS>
__device__ __forceinline__ void metadata_group(const int32_t* __restrict__ mapping, int num_tokens,
                                               int max_loras, const MetaOut& out, int g,
                                               MetaLds<THREADS>& sh) {
  constexpr int kWaves = THREADS / kWave;
  constexpr int kBlock = THREADS * kPerThread;
  int* const present = sh.present;
  int* const wave_below = sh.wave_below;
  int* const wave_members = sh.wave_members;
  int* const wave_none = sh.wave_none;
  int* const wave_scan = sh.wave_scan;
  int* const wave_runs = sh.wave_runs;
  int32_t* const staged = sh.staged;

  const int groups = max_loras + 1;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_index();
  for (int i = tid; i < groups; i += THREADS) present[i] = 0;
  __syncthreads();

  // Count pass: tokens in lower groups, members of g, occurring groups, and
  // (workgroup 0 only) the tokens that start a run of one adapter in batch
  // order: an adapter other than the previous token's.
  // Wave totals come straight from ballots (no cross-lane reduction).
  int grp[kPerThread];
  int wb = 0, wm = 0, wn = 0, wr = 0;
  for (int b0 = 0; b0 < num_tokens; b0 += kBlock) {
    const int t0 = b0 + tid * kPerThread;
    load_groups(mapping, num_tokens, max_loras, t0, grp);
    int prev = 0;  // group of token t0 - 1 (0: none, or no such token)
    if (g == 0 && t0 > 0 && t0 <= num_tokens) prev = group_of(mapping[t0 - 1], max_loras);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (grp[e] >= 0) present[grp[e]] = 1;  // benign: every writer stores 1
      wb += __popcll(__ballot(grp[e] >= 0 && grp[e] < g));
      wm += __popcll(__ballot(grp[e] == g));
      wn += __popcll(__ballot(grp[e] == 0));
      if (g == 0) {
        wr += __popcll(__ballot(grp[e] > 0 && grp[e] != prev));
        prev = grp[e];
      }
    }
  }
  if (lane == 0) {
    wave_below[wave] = wb;
    wave_members[wave] = wm;
    wave_none[wave] = wn;
    wave_runs[wave] = wr;
  }
  __syncthreads();
  int start = 0, total = 0, n_none = 0, runs = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    start += wave_below[w];
    total += wave_members[w];
    n_none += wave_none[w];
    runs += wave_runs[w];
  }

  if (g > 0 && total == 0) return;  // an adapter absent from the batch (uniform)

  // Every wave: g's slot among the adapters present and how many are present
  // (a few ballots; no barrier to share them).
  int k = 0, npresent = 0;
  for (int base = 0; base < groups; base += kWave) {
    const int i = base + lane;
    const bool p = i >= 1 && i < groups && present[i] != 0;
    k += __popcll(__ballot(p && i < g));
    npresent += __popcll(__ballot(p));
  }

  // An adapter's run of the padded order starts at pstart (group 0, no
  // adapter, has none).
  const bool has_run = g > 0;
  const int s_k = start - n_none;  // tokens of lower adapters
  const int pstart = round_up_tile(s_k + (kMetaTile - 1) * k);

  // The slot entries (group 0: the unused slots and the counts) and, past the
  // run's members, -1 up to the next run's start (for the last run, to the end
  // of its tile) and the tiles' adapter ids (-1 for a gap tile).  These depend
  // on the counts only, so they go out before the placing.
  if (g == 0) {
    for (int i = npresent + tid; i < max_loras; i += THREADS) {
      out.active_ids[i] = -1;
      out.counts[i] = 0;
      out.starts[i] = num_tokens;
    }
    if (tid == 0) *out.num_active = npresent;
    if (tid == 0) *out.num_runs = runs;
    if (tid == 0 && npresent == 0) *out.num_tiles = 0;
  } else {
    if (tid == 0) {
      out.active_ids[k] = g - 1;
      out.counts[k] = total;
      out.starts[k] = start;
    }
    const int run_end = round_up_tile(pstart + total);
    const bool last = k == npresent - 1;
    const int pnext = last ? run_end : round_up_tile(s_k + total + (kMetaTile - 1) * (k + 1));
    for (int i = pstart + total + tid; i < pnext; i += THREADS) out.tile_ids[i] = -1;
    for (int m = pstart / kMetaTile + tid; m < pnext / kMetaTile; m += THREADS)
      out.tile_lora[m] = m < run_end / kMetaTile ? g - 1 : -1;
    if (last && tid == 0) *out.num_tiles = run_end / kMetaTile;
  }

  // Place pass: member rank = members in earlier blocks + exclusive scan of the
  // per-thread member counts (thread order is token order within a block).  A
  // batch of one block reuses the groups already in registers.
  int placed = 0;
  for (int b0 = 0; total > 0 && b0 < num_tokens; b0 += kBlock) {
    const int t0 = b0 + tid * kPerThread;
    if (num_tokens > kBlock) load_groups(mapping, num_tokens, max_loras, t0, grp);
    // members among this thread's tokens, and up to and including this lane
    // (ballots with masked popcounts: no chain of cross-lane shuffles)
    const unsigned long long upto = lane == kWave - 1 ? ~0ull : (2ull << lane) - 1ull;
    int mine = 0, incl = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      mine += grp[e] == g ? 1 : 0;
      incl += __popcll(__ballot(grp[e] == g) & upto);
    }
    if (lane == kWave - 1) wave_scan[wave] = incl;
    __syncthreads();
    int before = 0, block_total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int n = wave_scan[w];
      before += w < wave ? n : 0;
      block_total += n;
    }
    // The block's members go to LDS in rank order, then out to both orders as
    // contiguous runs (consecutive lanes, consecutive words: whole lines rather
    // than one scattered word per member).
    int r = before + incl - mine;  // rank within the block of this thread's first member
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (grp[e] == g) staged[r++] = t0 + e;
    }
    __syncthreads();
    for (int i = tid; i < block_total; i += THREADS) {
      const int32_t t = staged[i];
      if (start + placed + i < num_tokens) {
        out.sorted[start + placed + i] = t;
        if (has_run) out.tile_ids[pstart + placed + i] = t;
      }
    }
    placed += block_total;
    if (b0 + kBlock < num_tokens) __syncthreads();  // wave_scan and staged are reused
  }
}

// The same, with LDS of its own.
template <int THREADS>
__device__ __forceinline__ void metadata_group(const int32_t* __restrict__ mapping, int num_tokens,
                                               int max_loras, const MetaOut& out, int g) {
  __shared__ MetaLds<THREADS> sh;
  metadata_group<THREADS>(mapping, num_tokens, max_loras, out, g, sh);
}

}  // namespace lora
