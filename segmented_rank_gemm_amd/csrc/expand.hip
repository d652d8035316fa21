// Expand step: y[t][off_s + n] = bf16( y[t][off_s + n] + sum_k buf[s][t][k] * B_s[l][n][k] )
// for every token t with adapter l, every slice s and column n < n_s, where
// buf[s][t][k] is the sum of the shrink's hidden-dimension parts.
//
// vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1": the summary names the
// expand kernel, and "Why do we need a new set of kernels" the ungrouped V1
// batch it must serve.  MLC-LLM issue "[Tracking] Multi-LoRA Serving",
// Overview: per-segment low-rank multiplication in one launch.  Several output
// slices per call cover fused projections (qkv, gate_up).
//
// gfx950 mapping.  The step is bound by the read-modify-write of y, so the
// layout is chosen for the y stream: a wave owns 16 grouped tokens of one
// adapter and walks 128-column chunks of one slice.  Per chunk it computes
// D = buf . B^T + y (M = 16 tokens, N = 16 columns per block, 8 blocks) with
// the MFMA's accumulator input set to y itself.  The N index of each block is
// permuted so that block b, MFMA column c is physical column 8c + b: lane
// (c, g) then holds 8 consecutive columns of tokens 4g..4g+3, which it loads
// and stores as one 16-byte vector per token, and each y instruction covers
// four rows of 256 contiguous bytes.  The fp32 buf row is split into
// hi = bf16(v) and lo = bf16(v - hi) placed side by side along K (K = 2r), so
// the bf16 matrix cores see buf to about 16 significant bits while B stays
// exact; products accumulate in fp32 and the single rounding to bf16 happens
// at the store (hardware round-to-nearest-even).

#include "device_common.hpp"

namespace lora {

constexpr int kExpandThreads = 256;
constexpr int kExpandWaves = kExpandThreads / kWave;
constexpr int kExpandCols = 128;   // columns per chunk: 8 MFMA blocks of 16
constexpr int kMaxSharedCpr = 16;  // longest column range (chunks) of the shared-B kernel

struct ExpandParams {
  const float* buf;
  int num_splits;
  // shared-B kernel: the parts already summed per row (the shrink's part
  // sums, same bits as summing buf here), or null: sum buf's parts
  const float* part_sum;
  const uint16_t* b[LORA_MAX_SLICES];
  int n[LORA_MAX_SLICES];
  int off[LORA_MAX_SLICES];
  int range_end[LORA_MAX_SLICES];  // running count of column ranges through slice s
                                   // (ranks 8, 16; the shared-B kernel derives its own)
  int num_slices;
  int chunks_per_range;            // 0: the shared-B kernel chooses it
  int num_cus;
  int ranges_by_cpr[kMaxSharedCpr + 1];  // shared-B: column ranges for c chunks per range
  int order_range_fastest;  // unit order: the column ranges of a tile consecutive
  uint16_t* y;
  int64_t ldy;
  const int32_t* sorted;
  const int32_t* active_ids;
  const int32_t* counts;
  const int32_t* starts;
  const int32_t* num_active;
  const int32_t* tile_ids;   // the padded grouped order (16-token tiles of one adapter)
  const int32_t* tile_lora;
  const int32_t* num_tiles;
  const int32_t* num_runs;   // same-adapter runs of the batch in token order
  int max_tiles;             // tiles the padded order may use
  int max_tokens;
  int max_loras;
};

// Rank-vector operand of one MFMA: hi parts for lane groups 0-1, lo for 2-3.
template <int RANK>
struct RankOperand;

template <>
struct RankOperand<8> {
  static constexpr int kSteps = 1;  // one 16x16x16 MFMA: K = 16 = 2 x rank
  i16x4 op[1];
};

template <int RANK>
struct RankOperand {
  static constexpr int kSteps = RANK / 16;  // 16x16x32 MFMAs: each covers 16 ranks, hi + lo
  bf16x8 op[RANK / 16];
};

// One chunk of one 16-token block: y of tokens 4*grp..4*grp+3, 8 columns each.
struct YBlock {
  u32x4 v[4];
};

// One 128-column chunk of B (128 rows of RANK bf16, 256*RANK contiguous
// bytes) as this lane loads it: 16-byte pieces lane, lane + 64, ... of the
// chunk, so that every load instruction reads 1 KB of whole cache lines.  The
// wave then passes the chunk through its own LDS region to reach the MFMA
// operand layout, in which lane (c, g) needs row 8c + b of every block b: read
// straight from global memory, each instruction would touch 16 lines for 8 or
// 16 bytes each.
template <int RANK>
struct BStage {
  static constexpr int kPieces = RANK / 4;  // 16-byte pieces per lane
  u32x4 v[kPieces];
};

// LDS slot of 16-byte piece pr of chunk row `row` (RANK / 8 pieces per row):
// row-major, with the low bits XOR-ed by a key taken from the row's high bits,
// so that the 16 lanes reading rows 8c + b (c = 0..15) of one block fall on 16
// different bank groups.  From rank 16 on the key is four bits of row / 8; at
// rank 8 (one piece per row, 8-byte reads whose half-wave passes pair lanes c
// and c + 8 on the same banks unless bit 3 of c enters the key) it is three
// bits of row / 16, and a 16-lane write of 16 consecutive rows stays one
// contiguous 256-byte block.  (With three bits of row / 8 at every rank, rows
// c and c + 8 shared their banks: 2.4 conflict cycles per LDS instruction on
// the prefill expand, 1.4 on the decode expand.)  The XOR only touches bits
// below the row's block index: a bijection on the region's 16 * RANK slots.
template <int RANK>
__device__ __forceinline__ int bslot(int row, int pr) {
  if constexpr (RANK == 8) return row ^ ((row >> 4) & 7);
  return (row * (RANK / 8) + pr) ^ ((row >> 3) & 15);
}

// MW = 16-token blocks per tile; every block shares the B operand loads.
//
// A workgroup unit is (tile of 16 positions of the padded grouped order, all
// of one adapter, slice s, column range of 4*cpr chunks); wave w takes chunks
// w, w+4, ... of the range, so the four waves stream neighbouring columns
// together.  The unit's token ids, its adapter and the tile count load in one
// round trip.  The rank operand of the tile (sum over the shrink's parts,
// split hi/lo, already in MFMA operand layout) is built once per unit into LDS
// and shared by the four waves.
template <int RANK, int MW>
__global__ __launch_bounds__(kExpandThreads) __attribute__((amdgpu_waves_per_eu(RANK <= 16 ? 2 : 1)))
void expand_kernel(ExpandParams p) {
  static_assert(MW == 1, "a tile of the padded grouped order holds 16 tokens");
  constexpr int kTile = 16 * MW;
  constexpr int kSteps = RankOperand<RANK>::kSteps;
  constexpr int kOpWords = RANK == 8 ? 2 : 4;  // 32-bit words per lane per MFMA step
  __shared__ uint32_t a_lds[MW][kSteps][kOpWords][kWave];
  __shared__ u32x4 b_lds[kExpandWaves][16 * RANK];  // one B chunk per wave

  const int lane = lane_id();
  const int wave = wave_index();
  const int c = lane & 15;   // MFMA row (token) for the buf operand, column for B / D
  const int grp = lane >> 4;
  const int khalf = grp & 1;  // which half of each 16-rank (or 8-rank) group
  const bool use_lo = grp >= 2;
  const int cpr = p.chunks_per_range;

  // Units are (tile of the padded grouped order, column range).  Small batches
  // take every tile the order may use, so that a unit's token ids, its tile's
  // adapter and the batch's tile count load together in one round trip
  // (units of tiles past the count do nothing).  Large batches read the tile
  // count first (one round trip for the whole walk) and take only the tiles in
  // use, so that every XCD's run of units has work.
  //
  // The walk: by default each XCD takes one contiguous run of units (tiles of
  // one adapter share its L2).  A large batch whose same-adapter runs in batch
  // order average at least half a tile (runs <= 2 * tiles) has tiles of
  // neighbouring y rows; for it a plain grid-strided walk, which keeps all
  // workgroups on one stretch of the grouped order and so on one region of y,
  // was 3-5% faster (gate_up and qkv shapes, 2-16 K tokens, request-run maps),
  // while on maps of scattered tokens it was 2-7% slower.  All workgroups read
  // the same two counts, so they agree on the walk.
  const int ranges = p.range_end[p.num_slices - 1];
  int tiles = p.max_tiles;
  bool strided = false;
  if (p.order_range_fastest) {
    const int nt = *p.num_tiles;
    const int nr = *p.num_runs;
    tiles = __builtin_amdgcn_readfirstlane(nt);
    strided = __builtin_amdgcn_readfirstlane(nr) <= 2 * tiles;
  }
  const int units = tiles * ranges;
  XcdWalk walk = xcd_walk(units, gridDim.x);
  if (strided) walk = XcdWalk{static_cast<int>(blockIdx.x), units, static_cast<int>(gridDim.x)};

  // Token ids of a unit's rows (the rank-operand row c and the output rows
  // 4*grp + j; -1 for a pad entry), its tile's adapter and the tile count.
  int ta[MW], td[MW][4], tlora = 0, tcount = 0;
  auto load_tokens = [&](int u) {
    const int m = p.order_range_fastest ? u / ranges : u % tiles;
    const int* ids = p.tile_ids + m * kTile;
    ta[0] = ids[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) td[0][j] = ids[4 * grp + j];
    tlora = p.tile_lora[m];
    tcount = *p.num_tiles;
  };
  if (walk.next < walk.end) load_tokens(walk.next);

  for (bool first = true; walk.next < walk.end; walk.next += walk.step, first = false) {
    const int u = walk.next;
    if (!first) load_tokens(u);
    const int m = p.order_range_fastest ? u / ranges : u % tiles;
    const int cr = p.order_range_fastest ? u % ranges : u / tiles;
    // (every load of the unit's first round trip goes out before the test: the
    // compiler would otherwise sink some below it)
    asm volatile("" : : "v"(ta[0]), "v"(td[0][0]), "v"(td[0][1]), "v"(td[0][2]), "v"(td[0][3]),
                 "v"(tlora), "v"(tcount));
    if (m >= tcount || tlora < 0 || tlora >= p.max_loras) continue;  // unused or gap tile

    int s = 0;
#pragma unroll
    for (int i = 0; i < LORA_MAX_SLICES - 1; ++i) s += (i < p.num_slices - 1 && cr >= p.range_end[i]) ? 1 : 0;
    int n_s = p.n[0], off_s = p.off[0], r_before = 0;
    const uint16_t* bslice = p.b[0];
#pragma unroll
    for (int i = 1; i < LORA_MAX_SLICES; ++i) {
      if (s == i) {
        n_s = p.n[i];
        off_s = p.off[i];
        r_before = p.range_end[i - 1];
        bslice = p.b[i];
      }
    }
    const int chunks_s = (n_s + kExpandCols - 1) / kExpandCols;
    const int range_begin = (cr - r_before) * cpr * kExpandWaves;
    const int range_end = min(chunks_s, range_begin + cpr * kExpandWaves);
    const int ch0 = range_begin + wave;  // this wave's chunks: ch0, ch0 + 4, ...

    // Loads are unconditional and never masked here: a lane whose row has no
    // adapter (or whose column is past the slice) reads a clamped, valid
    // location, and its results are simply not stored; the matrix-core rows
    // of such a token, and the columns of such a column, touch nothing else.
    // B chunk: piece q = lane + 64 i is piece q % (RANK/8) of chunk row
    // q / (RANK/8); rows past the slice's end read its last row (their columns
    // are never stored).
    constexpr int kRowPieces = RANK / 8;
    auto load_b = [&](const uint16_t* bmat, int ch, BStage<RANK>& bs) {
#pragma unroll
      for (int i = 0; i < BStage<RANK>::kPieces; ++i) {
        const int q = lane + kWave * i;
        const int row = ch * kExpandCols + q / kRowPieces;
        const int rowc = row < n_s ? row : n_s - 1;
        bs.v[i] = load16(bmat + static_cast<int64_t>(rowc) * RANK + 8 * (q % kRowPieces));
      }
    };
    u32x4* const bw = b_lds[wave];
    auto stage_b = [&](const BStage<RANK>& bs) {
#pragma unroll
      for (int i = 0; i < BStage<RANK>::kPieces; ++i) {
        const int q = lane + kWave * i;
        bw[bslot<RANK>(q / kRowPieces, q % kRowPieces)] = bs.v[i];
      }
    };
    const uint16_t* bmat0 = bslice + static_cast<int64_t>(tlora) * n_s * RANK;

    // y rows (a pad entry reads row 0 and is never stored)
    int64_t yrow[MW][4];
    bool dval[MW][4];
#pragma unroll
    for (int mb = 0; mb < MW; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dval[mb][j] = td[mb][j] >= 0 && td[mb][j] < p.max_tokens;
        yrow[mb][j] = static_cast<int64_t>(dval[mb][j] ? td[mb][j] : 0) * p.ldy + off_s;
      }

    auto load_y = [&](int ch, YBlock (&yb)[MW]) {
      const int col = ch * kExpandCols + 8 * c;
      const int colc = col < n_s ? col : n_s - 8;
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) yb[mb].v[j] = load16_stream(p.y + yrow[mb][j] + colc);
    };
    // First chunk: B, then y, then (below) the shrink's parts, all issued
    // unconditionally (a wave without a chunk in this range reads the range's
    // last one and stores nothing), so that the compiler's wait counts stay
    // exact and no load waits for another.
    const int chf = ch0 < range_end ? ch0 : range_end - 1;
    YBlock ycur[MW], ynext[MW];
    BStage<RANK> bnext;
    load_b(bmat0, chf, bnext);
    load_y(chf, ycur);

    // Rank operand, built cooperatively: item (mb, q) is one MFMA step of one
    // block, i.e. one register set of the wave; its lane (c, grp) sums the
    // parts of ranks [k0, k0 + kPer) of token row c.  Parts go in groups (16
    // for rank 8, else 8) whose loads are all issued before the first add; the
    // adds run in part order.  Part slots past the last re-read the group's
    // first and are masked.
    {
      constexpr int kPer = RANK == 8 ? 4 : 8;
      constexpr int kGroup = RANK == 8 ? 16 : 8;
      const int64_t plane = static_cast<int64_t>(p.num_slices) * p.max_tokens * RANK;
      for (int item = wave; item < MW * kSteps; item += kExpandWaves) {
        const int mb = item / kSteps;
        const int q = item - mb * kSteps;
        const int k0 = RANK == 8 ? 4 * khalf : 16 * q + 8 * khalf;
        const bool aval = ta[mb] >= 0 && ta[mb] < p.max_tokens;
        const float* src0 =
            p.buf + (static_cast<int64_t>(s) * p.max_tokens + (aval ? ta[mb] : 0)) * RANK + k0;
        float v[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) v[e] = 0.f;
        for (int sp0 = 0; sp0 < p.num_splits; sp0 += kGroup) {
          uint32_t pm[kGroup];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) pm[i] = opaque_mask(sp0 + i < p.num_splits);
          u32x4 w[kGroup][kPer / 4];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const int sp = sp0 + i < p.num_splits ? sp0 + i : sp0;
#pragma unroll
            for (int e4 = 0; e4 < kPer / 4; ++e4) w[i][e4] = load16(src0 + sp * plane + 4 * e4);
          }
#pragma unroll
          for (int i = 0; i < kGroup; ++i)
#pragma unroll
            for (int e4 = 0; e4 < kPer / 4; ++e4)
#pragma unroll
              for (int e = 0; e < 4; ++e) v[4 * e4 + e] += __uint_as_float(w[i][e4][e] & pm[i]);
        }
#pragma unroll
        for (int e = 0; e < kPer; e += 2) {
          const uint32_t hi = pack_bf16x2(v[e], v[e + 1]);
          a_lds[mb][q][e / 2][lane] =
              use_lo ? pack_bf16x2(v[e] - bf16_lo(hi), v[e + 1] - bf16_hi(hi)) : hi;
        }
      }
    }
    __syncthreads();
    RankOperand<RANK> a[MW];
#pragma unroll
    for (int mb = 0; mb < MW; ++mb)
#pragma unroll
      for (int q = 0; q < kSteps; ++q) {
        if constexpr (RANK == 8) {
          a[mb].op[q] = __builtin_bit_cast(i16x4, u32x2{a_lds[mb][q][0][lane], a_lds[mb][q][1][lane]});
        } else {
          a[mb].op[q] = __builtin_bit_cast(
              bf16x8, u32x4{a_lds[mb][q][0][lane], a_lds[mb][q][1][lane], a_lds[mb][q][2][lane],
                            a_lds[mb][q][3][lane]});
        }
      }
    __syncthreads();  // the next unit may overwrite a_lds

    // One pass over one chunk (its B in this wave's LDS region): acc =
    // y + buf . B^T, stored for the tile's rows.
    auto pass = [&](int ch) {
      const int col = ch * kExpandCols + 8 * c;  // first of this lane's 8 columns
      const bool col_ok = col < n_s;
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        f32x4 acc[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t w = ycur[mb].v[j][b >> 1];
            acc[b][j] = (b & 1) ? bf16_hi(w) : bf16_lo(w);
          }
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
#pragma unroll
          for (int q = 0; q < kSteps; ++q) {
            // lane (c, g): row 8c + b, ranks 16q + 8*khalf.. (rank 8: 4*khalf..)
            if constexpr (RANK == 8) {
              const u32x2 w = reinterpret_cast<const u32x2*>(bw + bslot<RANK>(8 * c + b, 0))[khalf];
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                  a[mb].op[q], __builtin_bit_cast(i16x4, w), acc[b], 0, 0, 0);
            } else {
              const u32x4 w = bw[bslot<RANK>(8 * c + b, 2 * q + khalf)];
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a[mb].op[q], __builtin_bit_cast(bf16x8, w), acc[b], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (col_ok && dval[mb][j]) {
            const u32x4 out = {pack_bf16x2(acc[0][j], acc[1][j]), pack_bf16x2(acc[2][j], acc[3][j]),
                               pack_bf16x2(acc[4][j], acc[5][j]), pack_bf16x2(acc[6][j], acc[7][j])};
            store16_stream(p.y + yrow[mb][j] + col, out);
          }
        }
      }
    };

    // (The wave's own LDS reads and writes stay in program order, so its B
    // region can be refilled right after a pass.)
    stage_b(bnext);
    if (ch0 < range_end) {  // wave-uniform
      // Steady state: the next chunk's loads are issued unconditionally before
      // this chunk's passes; the last chunk is peeled off.
      int ch = ch0;
      for (; ch + kExpandWaves < range_end; ch += kExpandWaves) {
        load_y(ch + kExpandWaves, ynext);
        load_b(bmat0, ch + kExpandWaves, bnext);
        pass(ch);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) ycur[mb] = ynext[mb];
        stage_b(bnext);
      }
      pass(ch);
    }
  }
}

// Ranks 32 and 64: the B operand of a chunk (8 or 16 KB) outweighs the y bytes
// of a 16-token block, so the four waves of a workgroup work on the same chunk
// and share its B.  A unit is (tile of up to 64 grouped tokens cut from one
// adapter's segment, slice s, range of cpr chunks); wave w owns rows 16w..16w+15
// of the tile.  Per chunk the workgroup loads B once, in whole-line 16-byte
// pieces, into a double-buffered XOR-swizzled LDS region (two chunks ahead);
// each wave keeps its y block (one chunk ahead) and its rank operand in
// registers.  Rows past the tile's end read the tile's first row and are
// never stored.
constexpr int kSharedTile = 64;

// Chunks per column range of the shared-B kernel, chosen for the batch at
// hand (its tile count is known only on the device).  Each XCD's workgroups
// take its run of units in rounds; a unit costs its chunks plus a start-up,
// in chunk times: half a chunk of fixed latency (token ids, first B chunk)
// plus the fetch of the shrink's parts for the tile's rows, which pass through
// the CU like the chunks' B and y (measured: the kernels are bound by what
// each unit fetches, cache hits included).  The choice minimises rounds *
// (chunks + start-up), ties to the longer range; on the down_proj (rank 64,
// 8 parts: start-up 3.2) and 70B qkv (rank 32, 6 parts: 1.7) batches it picks
// the fastest length measured.  Every lane computes the same value.
// (The search runs at every workgroup's start, so it avoids integer division:
// the range counts come from the host, and the rounds, integers below 2^20,
// are exact enough in fp32 less a margin well above its rounding error.)
template <int RANK, bool SUMS>
__device__ int shared_chunks_per_range(const ExpandParams& p, int tiles, int grid) {
  // bytes one chunk moves: its B rows, and its y columns of the tile read and written
  constexpr float kChunkBytes = kExpandCols * RANK * 2 + kSharedTile * kExpandCols * 2 * 2;
  const float startup =
      0.5f + static_cast<float>(kSharedTile * RANK * 4) *
                 static_cast<float>(SUMS ? 1 : p.num_splits) / kChunkBytes;
  const int slots = (grid < p.num_cus ? grid : p.num_cus) / kXcds;  // CUs per XCD at work
  const float inv_slots = 1.0f / static_cast<float>(slots > 0 ? slots : 1);
  int best = 8;
  float best_cost = 3.0e38f;
  for (int cpr = kMaxSharedCpr; cpr >= 2; --cpr) {
    const int per_xcd = (tiles * p.ranges_by_cpr[cpr] + kXcds - 1) / kXcds;
    const float cost =
        ceilf(static_cast<float>(per_xcd) * inv_slots - 1e-3f) * (static_cast<float>(cpr) + startup);
    if (cost < best_cost) {
      best_cost = cost;
      best = cpr;
    }
  }
  return best;
}

// Rank 32 fits three waves per SIMD (158 VGPRs), so three workgroups share a CU
// (70B qkv batch: 39.3 against 40.8 us); rank 64 would spill there and runs
// two: the six-part batch is built for two waves per SIMD (left to itself the
// compiler took 32 accumulator registers more than that allows), the other
// rank-64 builds fit two as they are.
// SUMS: the rank vectors come summed (p.part_sum), else from buf's parts,
// whose loads go out GROUP parts at a time (the sum is the same bits for any
// GROUP: it starts at +0 and adds the parts in order, and the masked parts
// past the last add +0 to a sum that is never -0).
template <int RANK, bool SUMS = false, int GROUP = (RANK == 64 ? 4 : 8)>
__global__ __launch_bounds__(kExpandThreads)
__attribute__((amdgpu_waves_per_eu(RANK == 32 ? 3 : GROUP > 4 ? 2 : 1)))
void expand_shared_kernel(ExpandParams p) {
  constexpr int kSteps = RANK / 16;
  constexpr int kRowPieces = RANK / 8;           // 16-byte pieces per B row
  constexpr int kPieces = 16 * RANK / kExpandThreads;  // per thread per chunk
  __shared__ SegmentTable tab;
  __shared__ u32x4 b_lds[2][16 * RANK];
  // per wave: the 16 rows' rank sums, row stride RANK + 4 floats (rows start
  // on different banks)
  constexpr int kRankStride = RANK + 4;
  __shared__ __attribute__((aligned(16))) float rank_lds[kExpandWaves][16 * kRankStride];

  build_segment_table<kSharedTile>(tab, p.active_ids, p.counts, p.starts, p.num_active,
                                   p.max_loras, p.max_tokens);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_index();
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int khalf = grp & 1;
  const bool use_lo = grp >= 2;
  // (the table's values are the same in every lane: read them as scalars)
  const int num_tiles = __builtin_amdgcn_readfirstlane(tab.num_tiles);
  const int cpr = p.chunks_per_range > 0 ? p.chunks_per_range
                                         : shared_chunks_per_range<RANK, SUMS>(p, num_tiles, gridDim.x);
  int range_end[LORA_MAX_SLICES];  // running count of column ranges through slice s
  {
    int ranges = 0;
#pragma unroll
    for (int s = 0; s < LORA_MAX_SLICES; ++s) {
      if (s < p.num_slices) ranges += ((p.n[s] + kExpandCols - 1) / kExpandCols + cpr - 1) / cpr;
      range_end[s] = ranges;
    }
  }
  const int nranges = range_end[p.num_slices - 1];
  const int units = num_tiles * nranges;

  for (XcdWalk walk = xcd_walk(units, gridDim.x); walk.next < walk.end; walk.next += walk.step) {
    const int u = walk.next;
    // (large batches: a tile's column ranges consecutive, as in the kernel above)
    const int m = p.order_range_fastest ? u / nranges : u % num_tiles;
    const int cr = p.order_range_fastest ? u % nranges : u / num_tiles;
    const Tile tile = resolve_tile<kSharedTile>(tab, m);

    int s = 0;
#pragma unroll
    for (int i = 0; i < LORA_MAX_SLICES - 1; ++i) s += (i < p.num_slices - 1 && cr >= range_end[i]) ? 1 : 0;
    int n_s = p.n[0], off_s = p.off[0], r_before = 0;
    const uint16_t* bslice = p.b[0];
#pragma unroll
    for (int i = 1; i < LORA_MAX_SLICES; ++i) {
      if (s == i) {
        n_s = p.n[i];
        off_s = p.off[i];
        r_before = range_end[i - 1];
        bslice = p.b[i];
      }
    }
    const int chunks_s = (n_s + kExpandCols - 1) / kExpandCols;
    const int ch0 = (cr - r_before) * cpr;
    const int nch = min(chunks_s, ch0 + cpr) - ch0;  // >= 1
    const uint16_t* bmat = bslice + static_cast<int64_t>(tile.lora) * n_s * RANK;

    // Token ids: the rank-operand row c and the output rows 4*grp + j of this
    // wave's block.
    const int r0 = 16 * wave;
    const int tfirst = tile_token(p.sorted, tile.first, tile.rows, 0, p.max_tokens);
    const int ta = tile_token(p.sorted, tile.first, tile.rows, r0 + c, p.max_tokens);
    int td[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      td[j] = tile_token(p.sorted, tile.first, tile.rows, r0 + 4 * grp + j, p.max_tokens);
    const int tsafe = tfirst >= 0 ? tfirst : 0;
    int64_t yrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      yrow[j] = static_cast<int64_t>(td[j] >= 0 ? td[j] : tsafe) * p.ldy + off_s;

    auto load_y = [&](int ch, YBlock& yb) {
      const int col = ch * kExpandCols + 8 * c;
      const int colc = col < n_s ? col : n_s - 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) yb.v[j] = load16_stream(p.y + yrow[j] + colc);
    };
    struct BPieces {
      u32x4 v[kPieces];
    };
    // piece q = tid + 256 i of the chunk: piece q % kRowPieces of row
    // q / kRowPieces; rows past the slice's end read its last row.
    auto load_b = [&](int ch, BPieces& bp) {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int q = tid + kExpandThreads * i;
        const int row = ch * kExpandCols + q / kRowPieces;
        const int rowc = row < n_s ? row : n_s - 1;
        bp.v[i] = load16(bmat + static_cast<int64_t>(rowc) * RANK + 8 * (q % kRowPieces));
      }
    };
    auto stage_b = [&](int b, const BPieces& bp) {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int q = tid + kExpandThreads * i;
        b_lds[b][bslot<RANK>(q / kRowPieces, q % kRowPieces)] = bp.v[i];
      }
    };

    const int last = ch0 + nch - 1;
    YBlock ya, yb;
    BPieces bp;
    load_y(ch0, ya);
    load_b(ch0, bp);

    // Rank operand of this wave's rows: step q, lane (c, g) holds ranks
    // 16q + 8*khalf .. +8 of row c, summed over the parts, as hi or lo bf16.
    // The sums are made in a layout where every lane loads different data
    // (lane (c, g4) sums ranks [kSpan g4, +kSpan) of row c; the operand layout
    // would load each value twice, for its hi and its lo lanes), with the loads
    // of kGroup parts issued before the adds (adds in part order), and reach
    // the operand layout through the wave's own LDS slice.
    RankOperand<RANK> a;
    {
      constexpr int kSpan = RANK / 4;              // ranks summed per lane
      constexpr int kLd = kSpan / 4;               // 16-byte loads per part
      constexpr int kGroup = GROUP;                 // parts per batch of loads
      const int g4 = lane >> 4;
      const int64_t plane = static_cast<int64_t>(p.num_slices) * p.max_tokens * RANK;
      const float* src0 = p.buf +
                          (static_cast<int64_t>(s) * p.max_tokens + (ta >= 0 ? ta : tsafe)) * RANK +
                          kSpan * g4;
      float v[kSpan];
#pragma unroll
      for (int e = 0; e < kSpan; ++e) v[e] = 0.f;
      if constexpr (SUMS) {  // one plane, already summed in this order
        const float* sum0 = p.part_sum +
                            (static_cast<int64_t>(s) * p.max_tokens + (ta >= 0 ? ta : tsafe)) * RANK +
                            kSpan * g4;
#pragma unroll
        for (int l = 0; l < kLd; ++l) {
          const u32x4 w = load16(sum0 + 4 * l);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * l + e] = __uint_as_float(w[e]);
        }
      }
      for (int sp0 = 0; !SUMS && sp0 < p.num_splits; sp0 += kGroup) {
        uint32_t pm[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) pm[i] = opaque_mask(sp0 + i < p.num_splits);
        u32x4 w[kGroup][kLd];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          const int sp = sp0 + i < p.num_splits ? sp0 + i : sp0;
#pragma unroll
          for (int l = 0; l < kLd; ++l) w[i][l] = load16(src0 + sp * plane + 4 * l);
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
#pragma unroll
          for (int l = 0; l < kLd; ++l)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * l + e] += __uint_as_float(w[i][l][e] & pm[i]);
      }
      float* sl = rank_lds[wave];
#pragma unroll
      for (int l = 0; l < kLd; ++l)
        *reinterpret_cast<f32x4*>(sl + c * kRankStride + kSpan * g4 + 4 * l) =
            f32x4{v[4 * l], v[4 * l + 1], v[4 * l + 2], v[4 * l + 3]};
      // (the wave's own slice, written and read in program order: LDS
      // operations of a wave complete in order; the fences keep the compiler
      // from moving the reads above the other lanes' writes)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int q = 0; q < kSteps; ++q) {
        const float* r8 = sl + c * kRankStride + 16 * q + 8 * khalf;
        const f32x4 lo4 = *reinterpret_cast<const f32x4*>(r8);
        const f32x4 hi4 = *reinterpret_cast<const f32x4*>(r8 + 4);
        const float t[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        uint32_t words[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t hi = pack_bf16x2(t[e], t[e + 1]);
          words[e / 2] = use_lo ? pack_bf16x2(t[e] - bf16_lo(hi), t[e + 1] - bf16_hi(hi)) : hi;
        }
        a.op[q] = __builtin_bit_cast(bf16x8, u32x4{words[0], words[1], words[2], words[3]});
      }
    }

    // acc = y + buf . B^T for one chunk from LDS buffer b, stored for the
    // wave's rows that hold a token and columns inside the slice.
    auto pass = [&](int b, int ch, const YBlock& y) {
      const int col = ch * kExpandCols + 8 * c;
      const bool col_ok = col < n_s;
      f32x4 acc[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = y.v[j][bb >> 1];
          acc[bb][j] = (bb & 1) ? bf16_hi(w) : bf16_lo(w);
        }
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
          const u32x4 w = b_lds[b][bslot<RANK>(8 * c + bb, 2 * q + khalf)];
          acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.op[q], __builtin_bit_cast(bf16x8, w),
                                                            acc[bb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (col_ok && td[j] >= 0) {
          const u32x4 out = {pack_bf16x2(acc[0][j], acc[1][j]), pack_bf16x2(acc[2][j], acc[3][j]),
                             pack_bf16x2(acc[4][j], acc[5][j]), pack_bf16x2(acc[6][j], acc[7][j])};
          store16_stream(p.y + yrow[j] + col, out);
        }
      }
    };

    // (The previous unit ended on a barrier after its last read of b_lds.)
    stage_b(0, bp);
    load_b(min(ch0 + 1, last), bp);
    __syncthreads();
    // Chunk i uses LDS buffer i % 2 and y set ya (even) or yb (odd); its B was
    // staged one chunk earlier and its y loaded one chunk earlier.  Loads never
    // run past the range's last chunk for y (B past it repeats the last chunk).
    int i = 0;
    for (; i + 2 < nch; i += 2) {
      load_y(ch0 + i + 1, yb);
      pass(0, ch0 + i, ya);
      stage_b(1, bp);
      load_b(min(ch0 + i + 2, last), bp);
      __syncthreads();
      load_y(ch0 + i + 2, ya);
      pass(1, ch0 + i + 1, yb);
      stage_b(0, bp);
      load_b(min(ch0 + i + 3, last), bp);
      __syncthreads();
    }
    if (i + 1 < nch) {
      load_y(ch0 + i + 1, yb);
      pass(0, ch0 + i, ya);
      stage_b(1, bp);
      __syncthreads();
      pass(1, ch0 + i + 1, yb);
      __syncthreads();
    } else {
      pass(0, ch0 + i, ya);
      __syncthreads();
    }
  }
}

template <int RANK>
hipError_t launch_expand_shared(const ExpandParams& p, int grid, hipStream_t stream) {
  if (p.part_sum) {
    grid = resident_grid<expand_shared_kernel<RANK, true>>(kExpandThreads, grid);
    hipLaunchKernelGGL((expand_shared_kernel<RANK, true>), dim3(grid), dim3(kExpandThreads), 0,
                       stream, p);
    return hipGetLastError();
  }
  // Rank 64 with 5 or 6 parts: all parts in one batch of loads, one round
  // trip instead of two (226 VGPRs, two waves per SIMD).  down_proj shape,
  // 16 adapters, 6 parts: 18.5 against 19.3 us at 2048 tokens, 76.4 against
  // 80.5 at 16384.
  if constexpr (RANK == 64) {
    if (p.num_splits > 4 && p.num_splits <= 6) {
      grid = resident_grid<expand_shared_kernel<RANK, false, 6>>(kExpandThreads, grid);
      hipLaunchKernelGGL((expand_shared_kernel<RANK, false, 6>), dim3(grid),
                         dim3(kExpandThreads), 0, stream, p);
      return hipGetLastError();
    }
  }
  grid = resident_grid<expand_shared_kernel<RANK>>(kExpandThreads, grid);
  hipLaunchKernelGGL((expand_shared_kernel<RANK>), dim3(grid), dim3(kExpandThreads), 0, stream, p);
  return hipGetLastError();
}

template <int RANK, int MW>
hipError_t launch_expand_rank(const ExpandParams& p, int grid, hipStream_t stream) {
  grid = resident_grid<expand_kernel<RANK, MW>>(kExpandThreads, grid);
  hipLaunchKernelGGL((expand_kernel<RANK, MW>), dim3(grid), dim3(kExpandThreads), 0, stream, p);
  return hipGetLastError();
}


hipError_t launch_expand(const float* buf, int num_splits, const uint16_t* const* lora_b,
                         const int32_t* slice_sizes, int num_slices, int rank, uint16_t* y,
                         int64_t ldy, const lora_meta_t& meta, int max_tokens, int max_loras,
                         int num_cus, const lora_expand_config_t* config, hipStream_t stream,
                         const float* part_sum) {
  ExpandParams p{};
  p.buf = buf;
  p.num_splits = num_splits;
  p.part_sum = rank >= 32 ? part_sum : nullptr;
  p.num_slices = num_slices;
  int64_t total_chunks = 0;
  int off = 0;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) {
    if (s < num_slices) {
      p.b[s] = lora_b[s];
      p.n[s] = slice_sizes[s];
      p.off[s] = off;
      off += slice_sizes[s];
      total_chunks += (slice_sizes[s] + kExpandCols - 1) / kExpandCols;
    } else {
      p.b[s] = lora_b[0];
      p.n[s] = 0;
      p.off[s] = off;
    }
  }
  // Ranks 8 and 16: chunks per wave in a workgroup unit (the unit spans 4x as
  // many).  Small batches: as many as still give every CU ~16 units, at most 8.
  // Large batches: 2, i.e. 1024-column ranges taken one after another along a
  // tile's row (see the unit order below), so that the workgroups in flight
  // hold few distinct y rows at a time (measured on the gate_up shape at 1-16 K
  // tokens and the qkv shape at 1-4 K: 2 was the fastest of 1, 2, 3, 4, 8
  // everywhere, 5% ahead of 8 on the 8 K-token prefill batch).  Ranks 32 and 64
  // (shared-B kernel, all waves on one chunk): the kernel chooses the range
  // length from the batch's tile count (0 here).
  const bool shared = rank >= 32;
  const bool large = max_tokens > 512;
  const int64_t tiles = shared ? (static_cast<int64_t>(max_tokens) + kSharedTile - 1) / kSharedTile + max_loras
                               : LORA_MAX_TILES(static_cast<int64_t>(max_tokens), max_loras);
  int64_t cpr = 0;
  if (!shared) {
    cpr = tiles * total_chunks / (static_cast<int64_t>(num_cus) * 16);
    cpr = cpr < 1 ? 1 : (cpr > 8 ? 8 : cpr);
    if (large) cpr = 2;
  }
  if (config && config->chunks_per_range > 0) cpr = config->chunks_per_range;
  p.chunks_per_range = static_cast<int>(cpr);
  // Large batches take the column ranges of a tile one after another, so an
  // XCD's workgroups sweep whole y rows of a few tiles at a time (better DRAM
  // page locality: measured 125 vs 128 us on the prefill batch); small ones
  // keep tiles next to each other (their few rows fit a single sweep anyway).
  p.order_range_fastest = large ? 1 : 0;
  if (config && config->range_fastest >= 0) p.order_range_fastest = config->range_fastest;
  // (shared-B kernel: the shortest range it may choose bounds the units)
  const int per_unit = shared ? (p.chunks_per_range > 0 ? p.chunks_per_range : 2)
                              : p.chunks_per_range * kExpandWaves;
  int ranges = 0;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) {
    if (s < num_slices) {
      const int chunks = (slice_sizes[s] + kExpandCols - 1) / kExpandCols;
      ranges += (chunks + per_unit - 1) / per_unit;
    }
    p.range_end[s] = ranges;
  }
  p.y = y;
  p.ldy = ldy;
  p.sorted = meta.sorted_token_ids;
  p.active_ids = meta.active_lora_ids;
  p.counts = meta.num_tokens_per_lora;
  p.starts = meta.lora_token_start;
  p.num_active = meta.num_active;
  p.tile_ids = meta.tile_token_ids;
  p.tile_lora = meta.tile_lora;
  p.num_tiles = meta.num_tiles;
  p.num_runs = meta.num_runs;
  p.max_tiles = LORA_MAX_TILES(max_tokens, max_loras);
  p.max_tokens = max_tokens;
  p.max_loras = max_loras;

  p.num_cus = num_cus;
  for (int c = 2; c <= kMaxSharedCpr; ++c) {
    int r = 0;
    for (int s = 0; s < num_slices; ++s) r += ((slice_sizes[s] + kExpandCols - 1) / kExpandCols + c - 1) / c;
    p.ranges_by_cpr[c] = r;
  }
  int64_t grid = tiles * ranges;
  // shared-B: two workgroups per CU at rank 64, three at rank 32 (one hides
  // another's unit start-up; the range choice counts rounds per CU, whose
  // fetch rate bounds them all)
  int64_t wg_per_cu = shared ? (rank == 32 ? 3 : 2) : 8;
  if (config && config->workgroups_per_cu > 0) wg_per_cu = config->workgroups_per_cu;
  const int64_t cap = static_cast<int64_t>(num_cus) * wg_per_cu;
  grid = grid < cap ? grid : cap;
  grid = (grid + kXcds - 1) / kXcds * kXcds;  // whole rounds over the XCDs
  switch (rank) {
    case 8: return launch_expand_rank<8, 1>(p, static_cast<int>(grid), stream);
    case 16: return launch_expand_rank<16, 1>(p, static_cast<int>(grid), stream);
    case 32: return launch_expand_shared<32>(p, static_cast<int>(grid), stream);
    default: return launch_expand_shared<64>(p, static_cast<int>(grid), stream);
  }
}

}  // namespace lora
