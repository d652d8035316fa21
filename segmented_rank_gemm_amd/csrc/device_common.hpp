// Device-side helpers shared by the gfx950 kernels of the multi-LoRA path:
// 16-byte vector types, bf16 <-> fp32 conversion, wave-level scans, and the
// per-workgroup segment table that maps a flat tile index onto an adapter's
// group of tokens.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_mi355x.h"

namespace lora {

constexpr int kWave = 64;

// Shrink work split (shared by every shrink kernel, so that a part's partial
// sums are the same bits whichever kernel computes them): 256-thread
// workgroups whose four waves take interleaved 64-element chunks of a part.
constexpr int kShrinkThreads = 256;
constexpr int kShrinkWaves = kShrinkThreads / kWave;
constexpr int kShrinkChunk = 64;  // hidden elements per wave step (two MFMA K-steps)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// MFMA operand types: 8 bf16 (16x16x32) and 4 x 16-bit (16x16x16, "1k" form).
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));

// Every buffer of the path lives in device global memory: say so, so that
// pointers that went through LDS or a select still compile to global_* (not
// flat_*) instructions.
#define LORA_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *(const LORA_GLOBAL u32x4*)(p);
}
__device__ __forceinline__ u32x2 load8(const void* p) {
  return *(const LORA_GLOBAL u32x2*)(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *(LORA_GLOBAL u32x4*)(p) = v; }

// 16 bytes per lane from global memory straight into LDS (gfx950's
// global_load_lds_dwordx4): lane i's bytes land at lds + 16 i, so one
// instruction fills 1 KB of LDS in lane order while each lane names its own
// source.  `lds` must be the same for every lane of the wave.  Completion is
// counted like any vector load (vmcnt); no VGPR holds the data.
__device__ __forceinline__ void load16_to_lds(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((LORA_GLOBAL void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

// Streamed data touched once (the y rows; x rows where one unit reads them):
// non-temporal hint, so it does not displace the adapter weights that every
// tile re-reads from L2.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load((const LORA_GLOBAL u32x4*)(p));
}
__device__ __forceinline__ void store16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, (LORA_GLOBAL u32x4*)(p));
}

// Device-coherent 16-byte accesses, for data that one workgroup of a launch
// hands to another: the store is written through to the level every XCD shares
// (each XCD has its own L2) and the load is served from there, never from a
// stale line of the reading XCD's L2 (cache policy sc1, the code the compiler
// emits for agent-scope atomic loads and stores, here on 16 bytes at once).
// Offsets are bytes from the resource's base; an access past `bytes` is
// dropped (store) or reads zero (load).  Word 3 is the gfx9 raw-buffer format.
constexpr int kCachePolicyCoherent = 16;  // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyCoherent);
}
__device__ __forceinline__ u32x2 load8_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCachePolicyCoherent);
}
__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCachePolicyCoherent);
}
// Streamed data written through to that level as well (sc1 with the
// non-temporal hint): no dirty line of it is left in an XCD's L2 when the
// kernel ends.
constexpr int kCachePolicyStreamCoherent = 18;  // sc1 | nt
__device__ __forceinline__ void store16_stream_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                        u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCachePolicyStreamCoherent);
}

// Low / high bf16 of a packed pair, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values rounded to bf16 (nearest, ties to even) and packed, `lo` in
// the low half; one hardware conversion on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x & (kWave - 1)); }

// Exclusive prefix sum over the wave's lanes of v >= 0, bit-sliced: one ballot
// per bit in use, each lane counting the set bits of the lanes below it
// (v_mbcnt).  No chain of cross-lane shuffles (a dependent shuffle costs about
// 0.1 us on this part).
__device__ __forceinline__ int wave_exclusive_sum(int v) {
  int s = 0;
  for (int b = 0; b < 31; ++b) {
    if (__ballot((v >> b) != 0) == 0) break;  // wave-uniform
    const unsigned long long m = __ballot((v >> b) & 1);
    const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
    s += below << b;
  }
  return s;
}

// Segment table: the active adapter slots of one batch (from the metadata
// step) cut into tiles of TILE consecutive grouped tokens.  A tile never spans
// two adapters.  Built by wave 0 of every workgroup; slot data that does not
// describe a range inside [0, max_tokens) is dropped, so a corrupted metadata
// buffer cannot send a kernel outside its arrays.
struct SegmentTable {
  int start[LORA_MAX_LORAS];     // first grouped position of the slot
  int count[LORA_MAX_LORAS];     // tokens of the slot (0 if dropped)
  int lora[LORA_MAX_LORAS];      // adapter id of the slot
  int tile_end[LORA_MAX_LORAS];  // inclusive running sum of tiles per slot
  int num_slots;
  int num_tiles;
};

template <int TILE>
__device__ void build_segment_table(SegmentTable& tab, const int32_t* __restrict__ active_ids,
                                    const int32_t* __restrict__ counts,
                                    const int32_t* __restrict__ starts,
                                    const int32_t* __restrict__ num_active, int max_loras,
                                    int max_tokens) {
  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    // Every slot array is written in full by the metadata step, so all loads
    // go out together with the slot count: one round trip.
    int na = *num_active;
    int cnt0 = 0, st0 = 0, id0 = 0;
    if (lane < max_loras) {
      cnt0 = counts[lane];
      st0 = starts[lane];
      id0 = active_ids[lane];
    }
    na = na < 0 ? 0 : (na > max_loras ? max_loras : na);
    int carry = 0;
    for (int base = 0; base < na; base += kWave) {
      const int i = base + lane;
      int cnt = cnt0, st = st0, id = id0;
      if (base > 0) {
        cnt = 0;
        if (i < na) {
          cnt = counts[i];
          st = starts[i];
          id = active_ids[i];
        }
      }
      const bool ok = i < na && id >= 0 && id < max_loras && cnt > 0 && st >= 0 &&
                      st <= max_tokens && cnt <= max_tokens - st;
      if (!ok) cnt = 0;
      const int nt = (cnt + TILE - 1) / TILE;
      const int incl = wave_exclusive_sum(nt) + nt;
      if (i < na) {
        tab.start[i] = st;
        tab.count[i] = cnt;
        tab.lora[i] = ok ? id : 0;
        tab.tile_end[i] = carry + incl;
      }
      carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) {
      tab.num_slots = na;
      tab.num_tiles = carry;
    }
  }
  __syncthreads();
}

// Slot holding flat tile m (0 <= m < num_tiles), the first slot whose running
// tile count exceeds m.  Must be called with the same m by all lanes of a wave.
__device__ __forceinline__ int find_slot(const SegmentTable& tab, int m) {
  const int lane = lane_id();
  for (int base = 0; base < tab.num_slots; base += kWave) {
    const int i = base + lane;
    const unsigned long long hit = __ballot(i < tab.num_slots && tab.tile_end[i] > m);
    if (hit) return base + __ffsll(static_cast<long long>(hit)) - 1;
  }
  return 0;  // unreachable for m < num_tiles
}

// Tile m resolved to its adapter and grouped-token range [first, first + rows).
struct Tile {
  int lora;
  int first;
  int rows;
};

template <int TILE>
__device__ __forceinline__ Tile resolve_tile(const SegmentTable& tab, int m) {
  const int slot = find_slot(tab, m);
  const int before = slot > 0 ? tab.tile_end[slot - 1] : 0;
  const int j = m - before;
  Tile t;
  t.lora = tab.lora[slot];
  t.first = tab.start[slot] + j * TILE;
  const int left = tab.count[slot] - j * TILE;
  t.rows = left < TILE ? left : TILE;
  return t;
}

// Slot table: the active adapter slots of one batch (from the metadata step)
// as ranges of grouped positions [start, end), plus the range of positions that
// have an adapter at all.  Kernels cut the grouped order into fixed tiles of
// consecutive positions, so a tile's token ids can be loaded before this table
// is known; the table then says which slot (adapter) each row belongs to.  A
// slot whose data does not describe a range inside [0, max_tokens) is dropped,
// so a corrupted metadata buffer cannot send a kernel outside its arrays.
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2),
// so workgroup b runs on XCD b % 8.  Unit streams are remapped so that each XCD
// takes one contiguous run of the natural unit order (consecutive tiles of one
// adapter, sharing its weights in that XCD's L2): workgroup b walks units
// xcd * per_xcd + slot, + slots_per_xcd, ... within its XCD's run.
constexpr int kXcds = 8;

// Compute units of the MI355X (gfx950): 256, in 8 XCDs of 32.  Grid sizes
// are a function of the size arguments and these constants only.
constexpr int kCus = 256;

// Clamp a persistent grid to the workgroups the device holds at once, so that
// every launched workgroup runs from the start: one queued behind the resident
// ones would begin its share of the units only when another ends, and a share
// of large units then finishes far behind the rest.  Whole rounds over the
// XCDs.  Host only.  The kernel's workgroups per CU (a property of its code:
// registers and LDS) are looked up once per process and kept; a failed lookup
// leaves the grid as it is.
// (One instantiation per kernel, so each kernel keeps its own value.)
template <auto Kernel>
inline int resident_grid(int threads, int grid) {
  static const int per_cu = [threads] {
    int v = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, Kernel, threads, 0) == hipSuccess ? v : 0;
  }();
  if (per_cu < 1) return grid;
  int64_t cap = static_cast<int64_t>(per_cu) * kCus / kXcds * kXcds;
  cap = cap < kXcds ? kXcds : cap;
  return grid < cap ? grid : static_cast<int>(cap);
}

struct XcdWalk {
  int next;  // next unit index, or >= end when done
  int end;
  int step;
};

// b: this workgroup's index among the `grid` workgroups of the walk (its
// launch index, or that less a multiple of kXcds workgroups placed before it)
__device__ __forceinline__ XcdWalk xcd_walk(int units, int grid, int b) {
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  const int slots = grid / kXcds;  // grid is a multiple of kXcds
  XcdWalk w;
  w.next = xcd * per_xcd + slot;
  w.end = min(units, (xcd + 1) * per_xcd);
  w.step = slots;
  return w;
}
__device__ __forceinline__ XcdWalk xcd_walk(int units, int grid) {
  return xcd_walk(units, grid, static_cast<int>(blockIdx.x));
}

// Loads below are issued unconditionally from addresses that are always valid
// (masked lanes are pointed at a clamped, in-bounds location) and masked
// afterwards.  A load inside a branch would force a wait for it at the branch's
// join; unconditional loads let every load of a step be in flight together.

// Token index of row `r` of a tile (grouped positions first .. first+rows-1),
// or -1 for rows past the tile or an index outside [0, max_tokens).  rows >= 1.
__device__ __forceinline__ int tile_token(const int32_t* __restrict__ sorted, int first, int rows,
                                          int r, int max_tokens) {
  const int t = sorted[first + (r < rows ? r : rows - 1)];
  return (r < rows && t >= 0 && t < max_tokens) ? t : -1;
}

// All-ones or all-zeros, hidden from the optimizer (an empty asm with a VGPR
// operand, no instruction): `v & mask` then cannot be turned back into a load
// under a branch, which would wait for the load at the branch's join.
__device__ __forceinline__ uint32_t opaque_mask(bool keep) {
  uint32_t m = keep ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return m;
}
__device__ __forceinline__ u32x4 masked(u32x4 v, bool keep) { return v & opaque_mask(keep); }
__device__ __forceinline__ u32x2 masked(u32x2 v, bool keep) { return v & opaque_mask(keep); }

// ints per (tile, output group) arrival counter of the part sums: 64 bytes
constexpr int kPartCounterInts = 16;

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

}  // namespace lora
