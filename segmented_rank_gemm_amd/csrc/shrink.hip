// Shrink step: buf_p[s][t][k] = scale * sum_{h in part p} x[t][h] * A_s[l][k][h]
// for every token t with adapter l, read through the grouped token order.
//
// vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1": the summary names the
// shrink kernel; "Kernel Code Change" item 2 is the gather of the input tokens
// through the token -> LoRA map.  MLC-LLM issue "[Tracking] Multi-LoRA
// Serving", Overview: one launch covers every segment, each with its own
// low-rank weights.
//
// gfx950 mapping.  A work unit is (tile of 16*MW grouped tokens of one
// adapter, part p of the hidden dimension).  Each unit is a dense
// (16*MW)-token x (S*r)-output contraction, computed on the matrix cores as
// D^T = A . x^T with v_mfma_f32_16x16x32_bf16: the M dimension is the S*r
// outputs (blocks of 16), N the tokens (blocks of 16), K the hidden dimension.
// Every wave holds all MW x NB accumulator blocks, so each 16-byte operand it
// fetches feeds MW (or NB) matrix-core ops.  The sum over K is order-free, so
// lane group g (lanes 16g..16g+15) feeds MFMA i of a 64-wide chunk with the
// elements [32i + 8g, 32i + 8g + 8) of that chunk for BOTH operands: one load
// instruction covers 64 contiguous bytes of each of 16 rows, and the two
// instructions of a row's 128-byte line are issued back to back.  The four waves of a
// workgroup take interleaved chunks of the part and are summed through LDS in a
// fixed order, so results are bit-identical run to run.  The grid is fixed by
// the size arguments; workgroups stride over the units of the actual batch.

#include "device_common.hpp"
#include "metadata_group.hpp"

namespace lora {

constexpr int kMaxFusedLoras = 16;  // adapter slots the fused prepare + shrink serves
constexpr int kMaxFusedGroups = kMaxFusedLoras + 1;

struct ShrinkParams {
  const uint16_t* x;
  int64_t ldx;
  int hidden;
  const uint16_t* a[LORA_MAX_SLICES];
  int num_slices;
  int rank;
  int rank_shift;  // log2(rank)
  float scale;
  float* buf;
  int num_splits;
  int split_len;  // hidden elements per part, a multiple of kShrinkChunk
  int num_groups; // output groups of up to NB 16-output blocks each
  const int32_t* sorted;
  const int32_t* active_ids;
  const int32_t* counts;
  const int32_t* starts;
  const int32_t* num_active;
  const int32_t* tile_ids;   // the padded grouped order (16-token tiles)
  const int32_t* tile_lora;
  const int32_t* num_tiles;
  int max_tiles;             // tiles the padded order may use
  int max_tokens;
  int max_loras;
  // fused prepare + shrink only: the map, the batch size, the metadata outputs
  // (written by the workgroups past shrink_grid), the shrink's own grid
  const int32_t* mapping;
  int num_tokens;
  int shrink_grid;
  MetaOut meta_out;
  // large batches, ranks 32 and 64, when the caller gives a workspace: each
  // (64-token tile, output group) counts its parts in at part_counters, and
  // the last one to arrive sums them into part_sum (null: off)
  int* part_counters;
  float* part_sum;
  uint32_t buf_bytes;  // bytes of buf (under 2^32 whenever part_sum is set)
};

// NB = number of 16-output blocks covering num_slices * rank outputs;
// MW = 16-token blocks per tile, all held by every wave so that each A operand
// fetched feeds MW matrix-core ops.
//
// SELF: the fused prepare + shrink launch for batches of at most 512 token
// slots and 16 adapter slots.  The workgroups past shrink_grid compute the
// metadata (one group each, the metadata kernel's code); the others do not
// wait for it: wave 0 reads the whole map once (8 ids per lane), counts each
// adapter's tokens with ballots and places its run of the padded grouped order
// (start round_up(S_k + 15 k, 16), as the metadata step does), and per unit
// finds the adapter whose run covers the unit's tile and that adapter's
// members of the tile by their rank in token order.  So the shrink learns its tile from the map in the
// round trip that would otherwise fetch it from the metadata, and the two
// steps share one launch.
template <int NB, int MW, bool SELF = false>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkParams p) {
  static_assert(MW == 1, "a tile of the padded grouped order holds 16 tokens");
  constexpr int kTile = 16 * MW;
  if constexpr (SELF) {
    if (static_cast<int>(blockIdx.x) >= p.shrink_grid) {  // workgroup-uniform
      metadata_group<kShrinkThreads>(p.mapping, p.num_tokens, p.max_loras, p.meta_out,
                                     static_cast<int>(blockIdx.x) - p.shrink_grid);
      return;
    }
  }
  __shared__ f32x4 red[kShrinkWaves][NB][kWave];
  __shared__ const uint16_t* slice_a[LORA_MAX_SLICES];  // per-lane slice lookup without
                                                        // indexing the argument block
  if (threadIdx.x < LORA_MAX_SLICES) slice_a[threadIdx.x] = p.a[threadIdx.x];
  __syncthreads();

  // Units over every tile the padded order may use (tile fastest), so that a
  // unit's tile is known before the batch's tile count arrives: the unit's
  // token ids, its adapter and the count load in one round trip, and units of
  // tiles past the count do nothing.
  const int num_tiles = p.max_tiles;
  const int units = num_tiles * p.num_splits * p.num_groups;

  const int lane = lane_id();
  const int wave = wave_index();
  const int col = lane & 15;  // token within a 16-token block (MFMA N index)
  const int grp = lane >> 4;  // lane group: K sub-range, and output rows 4*grp..4*grp+3
  const int nout = p.num_slices * p.rank;

  // SELF: every wave reads the whole map (8 tokens per lane, at most 2 KB) and
  // keeps, lane-indexed (lane g for group g <= max_loras < 64), each adapter's
  // count and the start of its run of the padded order (-1: absent); the four
  // waves count a quarter of the groups each (ballots) and share the counts
  // through LDS.  Per unit each wave finds its tile's token ids itself and
  // passes them between its lanes through its own LDS slice, so no wave waits
  // for another.  Ballots, lane reads and scalar loops only: a chain of
  // cross-lane shuffles costs ~0.1 us a step here.
  __shared__ int w_tile[SELF ? kShrinkWaves : 1][kTile];
  __shared__ int g_count[SELF ? kMaxFusedGroups : 1];
  const int groups = p.max_loras + 1;
  int mgrp[kPerThread];
  int vcount = 0, vstart = -1, tiles_self = 0;
  if constexpr (SELF) {
    load_groups(p.mapping, p.num_tokens, p.max_loras, lane * kPerThread, mgrp);
    for (int gi = 1 + wave; gi < groups; gi += kShrinkWaves) {
      int c = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) c += __popcll(__ballot(mgrp[e] == gi));
      if (lane == 0) g_count[gi] = c;
    }
    __syncthreads();
    vcount = lane >= 1 && lane < groups ? g_count[lane] : 0;
    int below = 0, present = 0, end = 0;  // tokens and adapters before group g
    for (int gi = 1; gi < groups; ++gi) {
      const int c = __builtin_amdgcn_readlane(vcount, gi);
      const int start = round_up_tile(below + (kTile - 1) * present);
      vstart = lane == gi ? (c > 0 ? start : -1) : vstart;
      if (c > 0) {
        end = round_up_tile(start + c);
        below += c;
        ++present;
      }
    }
    tiles_self = end / kTile;
  }

  for (XcdWalk walk = xcd_walk(units, SELF ? p.shrink_grid : static_cast<int>(gridDim.x));
       walk.next < walk.end; walk.next += walk.step) {
    const int u = walk.next;
    const int pg = u / num_tiles;  // (part, output group), group fastest
    const int m = u - pg * num_tiles;
    const int part = pg / p.num_groups;
    const int o0 = (pg - part * p.num_groups) * 16 * NB;  // first output of the group
    int tiles_used, tile_lora, tile_id;
    if constexpr (SELF) {
      // the adapter group whose run covers tile m (runs start on tile
      // boundaries, so the tile overlaps run g iff start_g <= 16 m < start_g + count_g)
      int hit = -1, hit_start = 0;
      for (int gi = 1; gi < groups; ++gi) {
        const int st = __builtin_amdgcn_readlane(vstart, gi);
        const int c = __builtin_amdgcn_readlane(vcount, gi);
        if (st >= 0 && kTile * m >= st && kTile * m < st + c) {
          hit = gi;
          hit_start = st;
        }
      }
      int* slot = w_tile[wave];
      if (lane < kTile) slot[lane] = -1;
      if (hit > 0) {
        // its members of rank j0 .. j0 + 15 in token order: a token's rank is
        // the number of the group's tokens in lower lanes (ballots) plus those
        // before it in its own lane
        const int j0 = kTile * m - hit_start;
        const unsigned long long lower = (1ull << lane) - 1ull;
        int r = 0;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) r += __popcll(__ballot(mgrp[e] == hit) & lower);
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          if (mgrp[e] == hit) {
            if (r >= j0 && r < j0 + kTile) slot[r - j0] = lane * kPerThread + e;
            ++r;
          }
        }
      }
      // (one wave's own LDS slice, written and read in program order: LDS
      // operations of a wave complete in order; the fence keeps the compiler
      // from moving the read above the other lanes' writes)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      tiles_used = tiles_self;
      tile_lora = hit > 0 ? hit - 1 : -1;
      tile_id = slot[col];
    } else {
      tiles_used = *p.num_tiles;
      tile_lora = p.tile_lora[m];
      tile_id = p.tile_ids[kTile * m + col];  // this lane's token column
      // (the three loads go out together: the compiler would otherwise sink the
      // tile's two below the test, a second round trip)
      asm volatile("" : : "v"(tile_id), "v"(tile_lora), "v"(tiles_used));
    }
    if (m >= tiles_used) continue;  // wave-uniform
    Tile tile;
    tile.lora = tile_lora >= 0 && tile_lora < p.max_loras ? tile_lora : 0;
    const int kbeg = part * p.split_len;
    const int kend = min(p.hidden, kbeg + p.split_len);

    // A-operand rows: output o = o0 + 16*nb + col (the MFMA M index of this
    // lane); outputs past the last are pointed at the last and masked.
    const uint16_t* arow[NB];
    uint32_t amask[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int o = o0 + 16 * nb + col;
      const bool ok = o < nout;
      const int oc = ok ? o : nout - 1;
      const int s = oc >> p.rank_shift;
      const int k = oc & (p.rank - 1);
      arow[nb] = slice_a[s] + (static_cast<int64_t>(tile.lora) * p.rank + k) * p.hidden;
      amask[nb] = opaque_mask(ok);
    }

    // One 64-element chunk of both operands, as loaded (masks are applied at
    // use, so a chunk's loads stay in flight until its MFMAs need them).
    // Lane group g, MFMA i <-> elements [32i + 8g, +8) of the chunk: one
    // instruction reads 64 contiguous bytes of each of 16 rows, and the two
    // instructions of a row's 128-byte line are issued back to back.
    struct Chunk {
      u32x4 x[MW][2];
      u32x4 a[NB][2];
      uint32_t kmask[2];  // pieces inside the part (all ones except in a tail chunk)
    };
    // A chunk that runs past the part's end re-reads a piece inside the row
    // and masks (kend is a multiple of 8, so a piece is wholly in or out): the
    // part's first piece, or for an empty part (kbeg >= hidden, possible when
    // num_splits * split_len > hidden) the row's first.
    const int ksafe = kbeg < kend ? kbeg : 0;
    auto piece = [&](int kc, int i, bool full, uint32_t& km) {
      const int k = kc + 32 * i + 8 * grp;
      if (full) {
        km = 0xFFFFFFFFu;
        return k;
      }
      km = opaque_mask(k < kend);
      return k < kend ? k : ksafe;
    };
    auto load_a = [&](int kc, Chunk& c) {
      const bool full = kc + kShrinkChunk <= kend;  // wave-uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = piece(kc, i, full, c.kmask[i]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) c.a[nb][i] = load16(arow[nb] + k);
      }
    };
    const uint16_t* xrow[MW];
    uint32_t xmask[MW];
    // x rows with the streaming hint: read once per unit, while the A rows
    // are re-read by every tile of the adapter (decode shrink 4.79 -> 4.62 us;
    // the large-batch kernels, whose x goes through LDS, did not move)
    auto load_x = [&](int kc, Chunk& c) {
      const bool full = kc + kShrinkChunk <= kend;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t km;
        const int k = piece(kc, i, full, km);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) c.x[mb][i] = load16_stream(xrow[mb] + k);
      }
    };

    // This wave's chunks: kc, kc + kStride, ... below kend.  Every load below
    // is issued unconditionally (a wave without a chunk reads a chunk at ksafe,
    // inside every row, and adds nothing), so the compiler's wait counts stay
    // exact and no load waits for a later one.  The token ids go first, then the first A
    // chunk (which does not depend on them), then the first x chunk.
    constexpr int kStride = kShrinkWaves * kShrinkChunk;
    int kc = kbeg + wave * kShrinkChunk;
    const int nw = kc < kend ? (kend - kc + kStride - 1) / kStride : 0;  // wave-uniform
    kc = kc < kend ? kc : ksafe;
    int tok[MW];
    tok[0] = tile_id >= 0 && tile_id < p.max_tokens ? tile_id : -1;  // -1: a pad entry
    Chunk c0, c1;
    load_a(kc, c0);
#pragma unroll
    for (int mb = 0; mb < MW; ++mb) {
      xrow[mb] = p.x + static_cast<int64_t>(tok[mb] >= 0 ? tok[mb] : 0) * p.ldx;
      xmask[mb] = opaque_mask(tok[mb] >= 0);
    }
    load_x(kc, c0);

    f32x4 acc[MW][NB];
#pragma unroll
    for (int mb = 0; mb < MW; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mma = [&](const Chunk& c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4 xv[MW];
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) xv[mb] = c.x[mb][i] & (xmask[mb] & c.kmask[i]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 av = c.a[nb][i] & amask[nb];
#pragma unroll
          for (int mb = 0; mb < MW; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv[mb]), acc[mb][nb],
                0, 0, 0);
        }
      }
    };

    // Double-buffered walk over this wave's chunks, alternating two register
    // sets (no copies, which would make the compiler wait for one set's loads
    // before reusing its registers); the scheduling barriers keep each chunk's
    // loads ahead of the previous chunk's matrix-core ops, which wait for that
    // chunk's data.
    if (nw > 0) {
      int j = 0;
      for (; j + 2 < nw; j += 2) {
        load_a(kc + (j + 1) * kStride, c1);
        load_x(kc + (j + 1) * kStride, c1);
        __builtin_amdgcn_sched_barrier(0);
        mma(c0);
        load_a(kc + (j + 2) * kStride, c0);
        load_x(kc + (j + 2) * kStride, c0);
        __builtin_amdgcn_sched_barrier(0);
        mma(c1);
      }
      if (j + 1 < nw) {
        load_a(kc + (j + 1) * kStride, c1);
        load_x(kc + (j + 1) * kStride, c1);
        __builtin_amdgcn_sched_barrier(0);
        mma(c0);
        mma(c1);
      } else {
        mma(c0);
      }
    }

    // Sum the four waves' partial sums in a fixed order, one 16-token block at a
    // time; wave w finishes the output blocks nb = w, w+4, ...
#pragma unroll
    for (int mb = 0; mb < MW; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[wave][nb][lane] = acc[mb][nb];
      __syncthreads();
      const int t = tok[mb];  // token of this lane's column `col`
      for (int nb = wave; nb < NB; nb += kShrinkWaves) {
        f32x4 v = red[0][nb][lane];
#pragma unroll
        for (int w = 1; w < kShrinkWaves; ++w) v += red[w][nb][lane];
        // D^T layout: this lane holds outputs o = o0 + 16*nb + 4*grp + j (j = 0..3)
        // of token column `col`; rank is a multiple of 8, so the four share a slice.
        const int o = o0 + 16 * nb + 4 * grp;
        if (t >= 0 && o < nout) {
          const int s = o >> p.rank_shift;
          const int k = o & (p.rank - 1);
          v *= p.scale;
          float* dst = p.buf +
                       ((static_cast<int64_t>(part) * p.num_slices + s) * p.max_tokens + t) * p.rank + k;
          store16(dst, __builtin_bit_cast(u32x4, v));
        }
      }
      __syncthreads();
    }
  }
}

// Large batches: the same contraction with both operands staged through LDS.
// A unit is (tile of 64 grouped tokens of one adapter, part, group of NB <= 8
// output blocks).  Per 64-element chunk the workgroup fetches the tile's 64 x
// rows and 16*NB A rows with full-line loads (8 lanes per 128-byte row line,
// every byte of every line used) into LDS, where the row's 16-byte pieces are
// XOR-swizzled by row so that the MFMA-layout reads (16 rows x 16 bytes per
// instruction) hit 16 distinct banks.  Two or four chunks are in flight in
// registers ahead of the one being computed; LDS is double-buffered, one barrier per
// chunk.  Wave w owns token block w (16 tokens) and all output blocks, so no
// cross-wave reduction is needed.
constexpr int kLdsTile = 64;  // tokens per tile (4 waves x 16)
// Chunks in flight in registers: four at four output blocks (down_proj,
// rank 64: 21.3-21.4 against 21.8-22.1 us), else two (measured at four: the
// gate_up prefill shape's two blocks 18.4 against 18.1 us, the 70B qkv
// shape's six 30.4 against 28.6 us); two with part sums (four would spill).
constexpr int lds_depth(int nb, bool sums) { return nb == 4 && !sums ? 4 : 2; }

// Three workgroups per CU (registers and LDS allow it up to NB = 6), so that a
// batch's units all run in one round.
template <int NB, bool SUMS = false, int DEPTH = lds_depth(NB, SUMS)>
__global__ __launch_bounds__(kShrinkThreads) __attribute__((amdgpu_waves_per_eu(NB <= 6 ? 3 : 2)))
void shrink_lds_kernel(ShrinkParams p) {
  constexpr int kRows = kLdsTile + 16 * NB;       // x rows, then A rows
  constexpr int kJ = (kRows * 8 + kShrinkThreads - 1) / kShrinkThreads;  // pieces per thread
  constexpr int kLdsRows = kJ * (kShrinkThreads / 8);
  __shared__ SegmentTable tab;
  __shared__ u32x4 stage[2][kLdsRows * 8];
  __shared__ const uint16_t* slice_a[LORA_MAX_SLICES];
  __shared__ int last_part;

  if (threadIdx.x < LORA_MAX_SLICES) slice_a[threadIdx.x] = p.a[threadIdx.x];
  build_segment_table<kLdsTile>(tab, p.active_ids, p.counts, p.starts, p.num_active, p.max_loras,
                                p.max_tokens);
  const int num_tiles = tab.num_tiles;
  const int units = num_tiles * p.num_splits * p.num_groups;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_index();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int nout = p.num_slices * p.rank;
  const int piece = tid & 7;     // this thread's 16-byte piece of every row it loads
  const int row0 = tid >> 3;     // rows row0 + 32 j, j < kJ

  // Part sums (p.part_sum set): parts are written with device-coherent
  // stores; once all of a unit's have completed, one thread counts the part
  // in at its (tile, output group) counter, and the workgroup that brings the
  // count to num_splits reads every part of that tile and group back
  // (device-coherent loads: other XCDs wrote them), sums them in part order
  // from +0, as the expand does, into part_sum and returns the counter to
  // zero.  Integer counters only: the sum is the same bits whichever unit is
  // last.  (A sum that starts at +0 is never -0, so the +0 the expand adds for
  // the parts past the last of its batch changes no bit.)
  constexpr bool sums = SUMS;  // p.part_sum and p.part_counters set
  const __amdgpu_buffer_rsrc_t rbuf = buffer_rsrc(p.buf, sums ? p.buf_bytes : 0u);
  auto store_part = [&](int64_t e, f32x4 v) {
    if constexpr (sums)
      store16_coherent(rbuf, static_cast<uint32_t>(e * 4), __builtin_bit_cast(u32x4, v));
    else
      store16(p.buf + e, __builtin_bit_cast(u32x4, v));
  };
  auto count_in = [&](int m, int o0, const Tile& tile) {
    if constexpr (!sums) return;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's part stores have completed
    __syncthreads();
    int* const ctr = p.part_counters + (m * p.num_groups + o0 / (16 * NB)) * kPartCounterInts;
    if (tid == 0)
      last_part = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  p.num_splits - 1;
    __syncthreads();
    if (!last_part) return;  // workgroup-uniform
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // thread: tile row tid / 4, quads (tid % 4) + 4 k (k < NB) of the group's
    // 4 NB quads of 4 outputs; parts in batches (four, or two above four
    // blocks, within the registers), every load of a batch in flight before
    // its adds
    const int t = tile_token(p.sorted, tile.first, tile.rows, tid >> 2, p.max_tokens);
    if (t < 0) return;  // a pad row (no barrier follows)
    const int64_t plane = static_cast<int64_t>(p.num_slices) * p.max_tokens * p.rank;
    int64_t e0[NB];
    bool ok[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int o = o0 + 4 * ((tid & 3) + 4 * k);
      ok[k] = o < nout;
      const int oc = ok[k] ? o : o0;
      e0[k] = (static_cast<int64_t>(oc >> p.rank_shift) * p.max_tokens + t) * p.rank +
              (oc & (p.rank - 1));
    }
    f32x4 v[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kBatch = NB <= 4 ? 4 : 2;
    for (int sp0 = 0; sp0 < p.num_splits; sp0 += kBatch) {
      u32x4 w[kBatch][NB];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int sp = sp0 + i < p.num_splits ? sp0 + i : sp0;
#pragma unroll
        for (int k = 0; k < NB; ++k)
          w[i][k] = load16_coherent(rbuf, static_cast<uint32_t>((e0[k] + sp * plane) * 4));
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (sp0 + i < p.num_splits)  // uniform
#pragma unroll
          for (int k = 0; k < NB; ++k) v[k] += __builtin_bit_cast(f32x4, w[i][k]);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (ok[k]) store16(p.part_sum + e0[k], __builtin_bit_cast(u32x4, v[k]));
  };

  for (XcdWalk walk = xcd_walk(units, gridDim.x); walk.next < walk.end; walk.next += walk.step) {
    const int u = walk.next;
    const int pg = u / num_tiles;
    const int m = u - pg * num_tiles;
    const int part = pg / p.num_groups;
    const int o0 = (pg - part * p.num_groups) * 16 * NB;
    const Tile tile = resolve_tile<kLdsTile>(tab, m);
    const int kbeg = part * p.split_len;
    const int kend = min(p.hidden, kbeg + p.split_len);
    if (kbeg >= kend) {
      // an empty part still owes its (zero) contribution
      const int t = tile_token(p.sorted, tile.first, tile.rows, 16 * wave + col, p.max_tokens);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int o = o0 + 16 * nb + 4 * grp;
        if (t >= 0 && o < nout) {
          const int64_t e = ((static_cast<int64_t>(part) * p.num_slices + (o >> p.rank_shift)) *
                             p.max_tokens + t) * p.rank + (o & (p.rank - 1));
          store_part(e, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
      count_in(m, o0, tile);
      continue;
    }

    const int t = tile_token(p.sorted, tile.first, tile.rows, 16 * wave + col, p.max_tokens);
    // Source row of each piece this thread loads: x rows of the tile's tokens
    // (a row without a token reads row 0: its outputs are never stored), then
    // A rows of the group's outputs (an output past the last reads the last).
    const uint16_t* src[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int r = row0 + 32 * j;
      if (r < kLdsTile) {
        const int t = tile_token(p.sorted, tile.first, tile.rows, r, p.max_tokens);
        src[j] = p.x + static_cast<int64_t>(t >= 0 ? t : 0) * p.ldx;
      } else {
        int o = o0 + (r - kLdsTile);
        o = o < nout ? o : nout - 1;
        src[j] = slice_a[o >> p.rank_shift] +
                 (static_cast<int64_t>(tile.lora) * p.rank + (o & (p.rank - 1))) * p.hidden;
      }
    }
    // Chunk c of the part (clamped to the last, so that every load is issued
    // unconditionally and the compiler's wait counts stay exact).  A piece
    // past the part's end reads the part's first piece instead; the x operand
    // of such a piece is zeroed when it is read from LDS, so it adds nothing.
    const int nchunks = (kend - kbeg + kShrinkChunk - 1) / kShrinkChunk;
    struct Staged {
      u32x4 v[kJ];
    };
    auto gload = [&](int c, Staged& st) {
      const int k = kbeg + (c < nchunks ? c : nchunks - 1) * kShrinkChunk + 8 * piece;
      const int kk = k < kend ? k : kbeg;
#pragma unroll
      for (int j = 0; j < kJ; ++j) st.v[j] = load16(src[j] + kk);
    };
    auto sstore = [&](int b, const Staged& st) {
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int r = row0 + 32 * j;
        stage[b][r * 8 + (piece ^ (r & 7))] = st.v[j];
      }
    };

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int b, int c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pc = 4 * i + grp;  // 16-byte piece holding elements [32i + 8*grp, +8)
        const int xr = 16 * wave + col;
        const uint32_t in = kbeg + c * kShrinkChunk + 8 * pc < kend ? 0xFFFFFFFFu : 0u;
        const u32x4 xv = stage[b][xr * 8 + (pc ^ (xr & 7))] & in;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int ar = kLdsTile + 16 * nb + col;
          const u32x4 av = stage[b][ar * 8 + (pc ^ (ar & 7))];
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv), acc[nb], 0, 0, 0);
        }
      }
    };

    // DEPTH chunks in flight in registers ahead of the one computed (chunk j
    // in r[j % DEPTH], LDS buffer j % 2).  Chunks go in groups of DEPTH with
    // one exit test per group, so that every path into a wait has the same
    // loads outstanding; loads past the last chunk repeat it into registers
    // no one stores any more.  (The previous unit ended on a barrier after
    // its last read of stage.)
    static_assert(DEPTH >= 2 && DEPTH % 2 == 0, "chunk c sits in LDS buffer c % 2");
    Staged r[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) gload(i, r[i]);
    sstore(0, r[0]);
    gload(DEPTH, r[0]);
    __syncthreads();
    int c = 0;
    for (; c + DEPTH <= nchunks; c += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        compute(i & 1, c + i);
        sstore((i + 1) & 1, r[(i + 1) % DEPTH]);
        gload(c + i + 1 + DEPTH, r[(i + 1) % DEPTH]);
        __syncthreads();
      }
    }
    // the last nchunks % DEPTH chunks: chunk c is in buffer 0, the rest in
    // registers
#pragma unroll
    for (int i = 0; i < DEPTH - 1; ++i) {
      if (c + i >= nchunks) break;  // uniform
      compute(i & 1, c + i);
      if (c + i + 1 < nchunks) sstore((i + 1) & 1, r[(i + 1) % DEPTH]);
      __syncthreads();
    }

    // D^T layout: this lane holds outputs o0 + 16*nb + 4*grp + j (j = 0..3) of
    // token 16*wave + col of the tile; rank is a multiple of 8, so the four
    // share a slice.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int o = o0 + 16 * nb + 4 * grp;
      if (t >= 0 && o < nout) {
        const int64_t e = ((static_cast<int64_t>(part) * p.num_slices + (o >> p.rank_shift)) *
                           p.max_tokens + t) * p.rank + (o & (p.rank - 1));
        store_part(e, acc[nb] * p.scale);
      }
    }
    count_in(m, o0, tile);
  }
}

// Batch-order LDS shrink: the first launch of the step for large batches made
// of request runs.  Tile m is tokens [64m, 64m + 64) in batch order, so its x
// rows follow from m and no grouping is needed before the loads; the
// workgroups past shrink_grid compute the metadata in the same launch (the
// metadata kernel's per-group code).  Each adapter present in the tile is one
// pass of the LDS-staged kernel's chunk loop over x and that adapter's A rows,
// storing the outputs of the tile's tokens that have that adapter; a tile's
// first adapter and its others are separate units (two per tile and part),
// so a tile that straddles two requests takes two workgroups, not twice one's
// time.  A token's outputs are the same bits as the grouped kernel's: the same
// chunks, the same matrix-core sequence per token (a column of the product
// depends only on its own x row).  A tile with k adapters streams its x rows k
// times, so this suits batches whose tiles hold one or two adapters (PR13096's
// V1 batches of whole requests), not maps drawn per token.
template <int NB>
__global__ __launch_bounds__(kShrinkThreads) __attribute__((amdgpu_waves_per_eu(NB <= 6 ? 3 : 2)))
void shrink_batch_kernel(ShrinkParams p) {
  // The metadata workgroups come first (dispatched first, so they run beside
  // the shrink, not after it when the shrink fills the CUs), padded to whole
  // rounds over the XCDs so that the shrink's workgroups keep their XCDs.
  const int meta_wgs = (p.max_loras + 1 + kXcds - 1) / kXcds * kXcds;
  if (static_cast<int>(blockIdx.x) < meta_wgs) {  // workgroup-uniform
    if (static_cast<int>(blockIdx.x) <= p.max_loras)
      metadata_group<kShrinkThreads>(p.mapping, p.num_tokens, p.max_loras, p.meta_out,
                                     static_cast<int>(blockIdx.x));
    return;
  }
  constexpr int kRows = kLdsTile + 16 * NB;       // x rows, then A rows
  constexpr int kJ = (kRows * 8 + kShrinkThreads - 1) / kShrinkThreads;  // pieces per thread
  constexpr int kLdsRows = kJ * (kShrinkThreads / 8);
  __shared__ u32x4 stage[2][kLdsRows * 8];
  __shared__ const uint16_t* slice_a[LORA_MAX_SLICES];
  if (threadIdx.x < LORA_MAX_SLICES) slice_a[threadIdx.x] = p.a[threadIdx.x];
  __syncthreads();

  const int tiles = (p.num_tokens + kLdsTile - 1) / kLdsTile;
  const int units = 2 * tiles * p.num_splits * p.num_groups;  // (tile, first adapter or the rest)
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_index();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int nout = p.num_slices * p.rank;
  const int piece = tid & 7;
  const int row0 = tid >> 3;

  for (XcdWalk walk = xcd_walk(units, p.shrink_grid, static_cast<int>(blockIdx.x) - meta_wgs);
       walk.next < walk.end; walk.next += walk.step) {
    const int u = walk.next >> 1;
    const bool rest = (walk.next & 1) != 0;  // the tile's adapters after its first
    const int pg = u / tiles;
    const int m = u - pg * tiles;
    const int part = pg / p.num_groups;
    const int o0 = (pg - part * p.num_groups) * 16 * NB;
    const int t0 = m * kLdsTile;  // < num_tokens
    const int kbeg = part * p.split_len;
    const int kend = min(p.hidden, kbeg + p.split_len);
    // this lane's token (MFMA N index) and its adapter; lane L of every wave
    // also holds the adapter of tile row L, so every wave sees the tile's set
    const int tm = t0 + 16 * wave + col;
    const int lm = tm < p.num_tokens ? group_of(p.mapping[tm], p.max_loras) - 1 : -1;
    const int lr = t0 + lane < p.num_tokens ? group_of(p.mapping[t0 + lane], p.max_loras) - 1 : -1;
    auto store_out = [&](int nb, f32x4 v) {
      const int o = o0 + 16 * nb + 4 * grp;
      if (o < nout) {
        float* dst = p.buf + ((static_cast<int64_t>(part) * p.num_slices + (o >> p.rank_shift)) *
                              p.max_tokens + tm) * p.rank + (o & (p.rank - 1));
        store16(dst, __builtin_bit_cast(u32x4, v));
      }
    };
    if (kbeg >= kend) {
      // an empty part still owes its (zero) contribution
      if (lm >= 0 && !rest)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) store_out(nb, f32x4{0.f, 0.f, 0.f, 0.f});
      continue;
    }
    const int nchunks = (kend - kbeg + kShrinkChunk - 1) / kShrinkChunk;
    // x rows: the tile's tokens (a row past the batch reads the tile's first)
    const uint16_t* src[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int r = row0 + 32 * j;
      if (r < kLdsTile) src[j] = p.x + static_cast<int64_t>(t0 + r < p.num_tokens ? t0 + r : t0) * p.ldx;
    }
    // The x pieces of the first two chunks go out right behind the map: they
    // do not depend on the tile's adapters (the first pass below then loads
    // only its A pieces for those chunks).  Pieces j < kLdsTile / 32 are x rows.
    struct Staged {
      u32x4 v[kJ];
    };
    auto chunk_k = [&](int c) {
      const int k = kbeg + (c < nchunks ? c : nchunks - 1) * kShrinkChunk + 8 * piece;
      return k < kend ? k : kbeg;
    };
    Staged ra, rb;
#pragma unroll
    for (int j = 0; j < kLdsTile / 32; ++j) {
      ra.v[j] = load16(src[j] + chunk_k(0));
      rb.v[j] = load16(src[j] + chunk_k(1));
    }
    bool x_in_flight = true;
    // the tile's adapters, lowest lane first (the same order in every wave):
    // the first, or all the others
    uint64_t pending = __ballot(lr >= 0);
    if (pending != 0) {
      const int first = __builtin_amdgcn_readlane(lr, static_cast<int>(__builtin_ctzll(pending)));
      pending = rest ? pending & ~__ballot(lr == first) : __ballot(lr == first);
    }
    while (pending != 0) {  // workgroup-uniform
      const int l = __builtin_amdgcn_readlane(lr, static_cast<int>(__builtin_ctzll(pending)));
      pending &= ~__ballot(lr == l);
      // A rows of adapter l for the group's outputs (past the last: the last)
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int r = row0 + 32 * j;
        if (r >= kLdsTile) {
          int o = o0 + (r - kLdsTile);
          o = o < nout ? o : nout - 1;
          src[j] = slice_a[o >> p.rank_shift] +
                   (static_cast<int64_t>(l) * p.rank + (o & (p.rank - 1))) * p.hidden;
        }
      }
      // the chunk loop of shrink_lds_kernel (its first two chunks' x already
      // in flight on the first pass)
      auto gload = [&](int c, Staged& st) {
        const int kk = chunk_k(c);
#pragma unroll
        for (int j = 0; j < kJ; ++j) st.v[j] = load16(src[j] + kk);
      };
      auto sstore = [&](int b, const Staged& st) {
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const int r = row0 + 32 * j;
          stage[b][r * 8 + (piece ^ (r & 7))] = st.v[j];
        }
      };
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto compute = [&](int b, int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int pc = 4 * i + grp;
          const int xr = 16 * wave + col;
          const uint32_t in = kbeg + c * kShrinkChunk + 8 * pc < kend ? 0xFFFFFFFFu : 0u;
          const u32x4 xv = stage[b][xr * 8 + (pc ^ (xr & 7))] & in;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int ar = kLdsTile + 16 * nb + col;
            const u32x4 av = stage[b][ar * 8 + (pc ^ (ar & 7))];
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv), acc[nb], 0, 0, 0);
          }
        }
      };
      if (x_in_flight) {
#pragma unroll
        for (int j = kLdsTile / 32; j < kJ; ++j) {
          ra.v[j] = load16(src[j] + chunk_k(0));
          rb.v[j] = load16(src[j] + chunk_k(1));
        }
        x_in_flight = false;
      } else {
        gload(0, ra);
        gload(1, rb);
      }
      sstore(0, ra);
      gload(2, ra);
      __syncthreads();
      int c = 0;
      for (; c + 2 <= nchunks; c += 2) {
        compute(0, c);
        sstore(1, rb);
        gload(c + 3, rb);
        __syncthreads();
        compute(1, c + 1);
        sstore(0, ra);
        gload(c + 4, ra);
        __syncthreads();
      }
      if (c < nchunks) {
        compute(0, c);
        __syncthreads();
      }
      if (lm == l)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) store_out(nb, acc[nb] * p.scale);
    }
  }
}

template <int NB>
hipError_t launch_shrink_batch_nb(ShrinkParams p, int grid, hipStream_t stream) {
  const int meta_wgs = (p.max_loras + 1 + kXcds - 1) / kXcds * kXcds;
  // what stays resident beside the metadata workgroups
  const int resident = resident_grid<shrink_batch_kernel<NB>>(kShrinkThreads, 1 << 30);
  const int room = (resident - meta_wgs) / kXcds * kXcds;
  grid = grid < room ? grid : (room >= kXcds ? room : kXcds);
  p.shrink_grid = grid;
  const int total = meta_wgs + grid;
  hipLaunchKernelGGL((shrink_batch_kernel<NB>), dim3(total), dim3(kShrinkThreads), 0, stream, p);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_shrink_lds_nb(const ShrinkParams& p, int grid, hipStream_t stream) {
  if (p.part_sum) {
    grid = resident_grid<shrink_lds_kernel<NB, true>>(kShrinkThreads, grid);
    hipLaunchKernelGGL((shrink_lds_kernel<NB, true>), dim3(grid), dim3(kShrinkThreads), 0, stream,
                       p);
    return hipGetLastError();
  }
  grid = resident_grid<shrink_lds_kernel<NB>>(kShrinkThreads, grid);
  hipLaunchKernelGGL((shrink_lds_kernel<NB>), dim3(grid), dim3(kShrinkThreads), 0, stream, p);
  return hipGetLastError();
}

template <int NB, int MW>
hipError_t launch_shrink_nb(const ShrinkParams& p, int grid, hipStream_t stream) {
  grid = resident_grid<shrink_kernel<NB, MW>>(kShrinkThreads, grid);
  hipLaunchKernelGGL((shrink_kernel<NB, MW>), dim3(grid), dim3(kShrinkThreads), 0, stream, p);
  return hipGetLastError();
}

// Fused prepare + shrink: the shrink's grid (as resident as the kernel allows),
// then one workgroup per metadata group.
template <int NB>
hipError_t launch_prep_shrink_nb(ShrinkParams p, int grid, hipStream_t stream) {
  grid = resident_grid<shrink_kernel<NB, 1, true>>(kShrinkThreads, grid);
  p.shrink_grid = grid;
  const int total = grid + p.max_loras + 1;
  hipLaunchKernelGGL((shrink_kernel<NB, 1, true>), dim3(total), dim3(kShrinkThreads), 0, stream, p);
  return hipGetLastError();
}

template <int MW>
hipError_t launch_shrink_mw(const ShrinkParams& p, int nb, int grid, hipStream_t stream) {
  switch (nb) {
    case 1: return launch_shrink_nb<1, MW>(p, grid, stream);
    case 2: return launch_shrink_nb<2, MW>(p, grid, stream);
    case 3: return launch_shrink_nb<3, MW>(p, grid, stream);
    case 4: return launch_shrink_nb<4, MW>(p, grid, stream);
    case 5:
    case 6: return launch_shrink_nb<6, MW>(p, grid, stream);
    default: return launch_shrink_nb<8, MW>(p, grid, stream);
  }
}

// Output blocks per group: all of them up to 8 (128 outputs), else groups of 8.
int shrink_group_blocks(int nb_total) { return nb_total <= 8 ? nb_total : 8; }

// 16-token blocks per tile: one for small batches (register kernel, more tiles
// in flight, hidden split across the four waves), four (64-token tiles, the
// LDS-staged kernel) for larger ones.
int shrink_tile_blocks(int max_tokens, int nb) {
  if (max_tokens <= 512) return 1;
  return 4;  // the LDS-staged kernel (64-token tiles)
}

int shrink_split_len(int hidden, int num_splits) {
  const int per = (hidden + num_splits - 1) / num_splits;
  return (per + kShrinkChunk - 1) / kShrinkChunk * kShrinkChunk;
}

int shrink_grid(int max_tiles, int num_splits, int num_groups, int num_cus) {
  const int64_t units = static_cast<int64_t>(max_tiles) * num_splits * num_groups;
  const int64_t cap = static_cast<int64_t>(num_cus) * 8;
  const int64_t g = units < cap ? units : cap;
  return static_cast<int>((g + kXcds - 1) / kXcds * kXcds);  // whole rounds over the XCDs
}

static ShrinkParams shrink_params(const uint16_t* x, int64_t ldx, int hidden,
                                  const uint16_t* const* lora_a, int num_slices, int rank,
                                  float scale, float* buf, int num_splits, const lora_meta_t& meta,
                                  int max_tokens, int max_loras) {
  ShrinkParams p{};
  p.x = x;
  p.ldx = ldx;
  p.hidden = hidden;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) p.a[s] = s < num_slices ? lora_a[s] : lora_a[0];
  p.num_slices = num_slices;
  p.rank = rank;
  p.rank_shift = rank == 8 ? 3 : rank == 16 ? 4 : rank == 32 ? 5 : 6;
  p.scale = scale;
  p.buf = buf;
  p.num_splits = num_splits;
  p.split_len = shrink_split_len(hidden, num_splits);
  p.sorted = meta.sorted_token_ids;
  p.active_ids = meta.active_lora_ids;
  p.counts = meta.num_tokens_per_lora;
  p.starts = meta.lora_token_start;
  p.num_active = meta.num_active;
  p.tile_ids = meta.tile_token_ids;
  p.tile_lora = meta.tile_lora;
  p.num_tiles = meta.num_tiles;
  p.max_tiles = LORA_MAX_TILES(max_tokens, max_loras);
  p.max_tokens = max_tokens;
  p.max_loras = max_loras;
  const int nb_total = (num_slices * rank + 15) / 16;
  const int nb = shrink_group_blocks(nb_total);
  p.num_groups = (nb_total + nb - 1) / nb;
  return p;
}

static int shrink_nb(int num_slices, int rank) {
  return shrink_group_blocks((num_slices * rank + 15) / 16);
}

// Part sums (ShrinkParams.part_sum): large batches (the LDS-staged kernel's
// 64-token tiles, which are the shared-B expand's) at ranks 32 and 64, with
// more than one part.  Workspace: the arrival counters, one 64-byte slot per
// (tile, output group), then the summed plane [S][max_tokens][r] fp32.
static bool part_sums_apply(int max_tokens, int rank) { return max_tokens > 512 && rank >= 32; }

static int64_t part_counter_bytes(int max_tokens, int max_loras, int num_slices, int rank) {
  const int64_t tiles = (static_cast<int64_t>(max_tokens) + kLdsTile - 1) / kLdsTile + max_loras;
  const int nb_total = (num_slices * rank + 15) / 16;
  const int nb = shrink_group_blocks(nb_total);
  const int64_t groups = (nb_total + nb - 1) / nb;
  const int64_t bytes = tiles * groups * kPartCounterInts * static_cast<int64_t>(sizeof(int));
  return (bytes + 255) / 256 * 256;
}

int64_t part_sum_workspace_bytes(int max_tokens, int max_loras, int num_slices, int rank) {
  if (!part_sums_apply(max_tokens, rank)) return 0;
  return part_counter_bytes(max_tokens, max_loras, num_slices, rank) +
         static_cast<int64_t>(num_slices) * max_tokens * rank * static_cast<int64_t>(sizeof(float));
}

// The counters and the plane inside a workspace of part_sum_workspace_bytes;
// null when the sums do not apply to the call (one part, or buf past 4 GB).
void part_sum_layout(void* workspace, int max_tokens, int max_loras, int num_slices, int rank,
                     int num_splits, int** counters, float** plane) {
  *counters = nullptr;
  *plane = nullptr;
  const int64_t buf_bytes = static_cast<int64_t>(num_splits) * num_slices * max_tokens * rank * 4;
  if (!workspace || !part_sums_apply(max_tokens, rank) || num_splits < 2 ||
      buf_bytes >= (int64_t{1} << 32))
    return;
  *counters = static_cast<int*>(workspace);
  *plane = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    part_counter_bytes(max_tokens, max_loras, num_slices, rank));
}

hipError_t launch_shrink(const uint16_t* x, int64_t ldx, int hidden, const uint16_t* const* lora_a,
                         int num_slices, int rank, float scale, float* buf, int num_splits,
                         const lora_meta_t& meta, int max_tokens, int max_loras, int num_cus,
                         hipStream_t stream, int* part_counters, float* part_sum) {
  ShrinkParams p = shrink_params(x, ldx, hidden, lora_a, num_slices, rank, scale, buf,
                                 num_splits, meta, max_tokens, max_loras);
  const int nb = shrink_nb(num_slices, rank);
  const int mw = shrink_tile_blocks(max_tokens, nb);
  if (mw == 4 && part_sum && part_counters) {
    p.part_counters = part_counters;
    p.part_sum = part_sum;
    p.buf_bytes = static_cast<uint32_t>(static_cast<int64_t>(num_splits) * num_slices *
                                        max_tokens * rank * 4);
  }
  if (mw == 4) {
    // large batch: LDS-staged kernel, 64-token tiles, at most 3 workgroups per
    // CU, in whole rounds over the XCDs (and no more than are resident)
    const int64_t tiles = (static_cast<int64_t>(max_tokens) + kLdsTile - 1) / kLdsTile + max_loras;
    int64_t g = tiles * num_splits * p.num_groups;
    const int64_t cap = static_cast<int64_t>(num_cus) * 3;
    g = g < cap ? g : cap;
    const int grid = static_cast<int>((g + kXcds - 1) / kXcds * kXcds);
    switch (nb) {
      case 1: return launch_shrink_lds_nb<1>(p, grid, stream);
      case 2: return launch_shrink_lds_nb<2>(p, grid, stream);
      case 3: return launch_shrink_lds_nb<3>(p, grid, stream);
      case 4: return launch_shrink_lds_nb<4>(p, grid, stream);
      case 5:
      case 6: return launch_shrink_lds_nb<6>(p, grid, stream);
      default: return launch_shrink_lds_nb<8>(p, grid, stream);
    }
  }
  const int grid = shrink_grid(p.max_tiles, num_splits, p.num_groups, num_cus);
  return launch_shrink_mw<1>(p, nb, grid, stream);
}

hipError_t launch_metadata(const int32_t* mapping, int num_tokens, int max_tokens, int max_loras,
                           const lora_meta_t& meta, hipStream_t stream);

// Metadata and shrink of one batch.  Up to 512 token slots (the register
// kernel's sizes, one wave holding the whole map) and 16 adapter slots (the
// shrink workgroups loop over the groups): one fused launch.  Otherwise the
// metadata kernel, then the shrink.

bool token_shrink_fits(int max_tokens, int max_loras, int num_slices, int rank);
hipError_t launch_token_prep_shrink(const int32_t* mapping, int num_tokens, const uint16_t* x,
                                    int64_t ldx, int hidden, const uint16_t* const* lora_a,
                                    int num_slices, int rank, float scale, float* buf,
                                    int num_splits, const lora_meta_t& meta, int max_tokens,
                                    int max_loras, hipStream_t stream);

hipError_t launch_prep_shrink(const int32_t* mapping, int num_tokens, const uint16_t* x,
                              int64_t ldx, int hidden, const uint16_t* const* lora_a,
                              int num_slices, int rank, float scale, float* buf, int num_splits,
                              const lora_meta_t& meta, int max_tokens, int max_loras,
                              int num_cus, hipStream_t stream, int* part_counters,
                              float* part_sum, bool batch_order) {
  // few adapter outputs: the shrink in batch order (token_step.hip), which
  // needs no grouping before its loads
  if (token_shrink_fits(max_tokens, max_loras, num_slices, rank))
    return launch_token_prep_shrink(mapping, num_tokens, x, ldx, hidden, lora_a, num_slices, rank,
                                    scale, buf, num_splits, meta, max_tokens, max_loras, stream);
  const int nb = shrink_nb(num_slices, rank);
  if (batch_order && shrink_tile_blocks(max_tokens, nb) == 4) {
    // large batch of request runs: the batch-order LDS shrink beside the
    // metadata workgroups, one launch
    ShrinkParams p = shrink_params(x, ldx, hidden, lora_a, num_slices, rank, scale, buf,
                                   num_splits, meta, max_tokens, max_loras);
    p.mapping = mapping;
    p.num_tokens = num_tokens;
    p.meta_out = MetaOut{meta.sorted_token_ids, meta.active_lora_ids, meta.num_tokens_per_lora,
                         meta.lora_token_start, meta.num_active, meta.tile_token_ids,
                         meta.tile_lora, meta.num_tiles, meta.num_runs};
    const int64_t tiles = (static_cast<int64_t>(max_tokens) + kLdsTile - 1) / kLdsTile;
    int64_t g = tiles * num_splits * p.num_groups;
    const int64_t cap = static_cast<int64_t>(num_cus) * 3;
    g = g < cap ? g : cap;
    const int grid = static_cast<int>((g + kXcds - 1) / kXcds * kXcds);
    switch (nb) {
      case 1: return launch_shrink_batch_nb<1>(p, grid, stream);
      case 2: return launch_shrink_batch_nb<2>(p, grid, stream);
      case 3: return launch_shrink_batch_nb<3>(p, grid, stream);
      case 4: return launch_shrink_batch_nb<4>(p, grid, stream);
      case 5:
      case 6: return launch_shrink_batch_nb<6>(p, grid, stream);
      default: return launch_shrink_batch_nb<8>(p, grid, stream);
    }
  }
  if (shrink_tile_blocks(max_tokens, nb) != 1 || max_tokens > kWave * kPerThread ||
      max_loras > kMaxFusedLoras) {
    const hipError_t e = launch_metadata(mapping, num_tokens, max_tokens, max_loras, meta, stream);
    if (e != hipSuccess) return e;
    return launch_shrink(x, ldx, hidden, lora_a, num_slices, rank, scale, buf, num_splits, meta,
                         max_tokens, max_loras, num_cus, stream, part_counters, part_sum);
  }
  ShrinkParams p = shrink_params(x, ldx, hidden, lora_a, num_slices, rank, scale, buf, num_splits,
                                 meta, max_tokens, max_loras);
  p.mapping = mapping;
  p.num_tokens = num_tokens;
  p.meta_out = MetaOut{meta.sorted_token_ids, meta.active_lora_ids, meta.num_tokens_per_lora,
                       meta.lora_token_start, meta.num_active, meta.tile_token_ids,
                       meta.tile_lora, meta.num_tiles, meta.num_runs};
  const int grid = shrink_grid(p.max_tiles, num_splits, p.num_groups, num_cus);
  switch (nb) {
    case 1: return launch_prep_shrink_nb<1>(p, grid, stream);
    case 2: return launch_prep_shrink_nb<2>(p, grid, stream);
    case 3: return launch_prep_shrink_nb<3>(p, grid, stream);
    case 4: return launch_prep_shrink_nb<4>(p, grid, stream);
    case 5:
    case 6: return launch_prep_shrink_nb<6>(p, grid, stream);
    default: return launch_prep_shrink_nb<8>(p, grid, stream);
  }
}

}  // namespace lora
