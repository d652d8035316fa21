// Small batches in batch order: the shrink, and the whole step in one launch.
//
// vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1": the shrink and
// expand kernels over a V1 batch that is not grouped by LoRA id ("Why do we
// need a new set of kernels"), with a launch grid a CUDA graph can capture
// ("Kernel Code Change" item 1).  MLC-LLM issue "[Tracking] Multi-LoRA
// Serving", Overview: one launch covers every segment of the batch.
//
// The grouped kernels (shrink.hip, expand.hip) first need the grouping: a
// round trip for the tile's token ids before the first row of x or y can be
// requested.  On a small batch that round trip, and the launch that computes
// the grouping, are most of the time.  Here tiles are 16 consecutive tokens in
// batch order, so the rows a unit reads are known from its index alone, and a
// tile's tokens may belong to different adapters:
//
// * shrink: D^T = A_all . x^T over the outputs of EVERY adapter slot (M =
//   max_loras * S * r, in groups of up to 8 blocks of 16), N = the 16 tokens,
//   K = a part of the hidden dimension; each token keeps the outputs of its
//   own adapter.  The loads of x, A and the map go out together at the start.
//   The work split (parts, 64-element chunks, the four waves' interleave and
//   their sum in wave order) is that of the grouped small-batch shrink, so the
//   parts are the same bits; the extra adapters cost matrix-core time and
//   L2-hit A traffic, which is why this path is kept to max_loras*S*r <= 256.
// * expand (one-launch step): D = buf . B_l^T + y per adapter l present in the
//   tile, each token's rank operand masked to its own adapter, y in the MFMA
//   accumulator as in expand.hip; B for every adapter slot of the chunk is
//   fetched at the start with y.
//
// One-launch step.  Workgroups [0, shrink_grid) compute parts, the next
// expand_grid workgroups expand, and the last max_loras + 1 compute the
// metadata (the metadata kernel's code).  A shrink unit writes its part with
// device-coherent stores, waits for them to complete, and increments its
// tile's arrival counter; an expand unit fetches its ids, then (each after a
// hold-off that leaves the shrink units' loads the fetch path first) its y
// and B, then polls the counter until every part of its tile has arrived and
// reads the parts
// with device-coherent loads.  Workgroups are dispatched in index order on
// each XCD and every shrink workgroup precedes every expand workgroup, so a
// waiting expand unit never holds a slot a part it waits for still needs; the
// wait is nevertheless bounded (wait_polls), and a unit that runs out of polls
// computes its tile's parts itself (the same code, the same bits) instead.
// Counters are integers only (no floating-point atomics): the results are the
// same bits whatever the order of arrival.  The counters return to zero by the
// end of every launch: each expand unit counts itself out after its wait, and
// the last one of a tile subtracts what the launch added.

#include <mutex>

#include "device_common.hpp"
#include "metadata_group.hpp"

namespace lora {

int shrink_split_len(int hidden, int num_splits);  // shrink.hip

constexpr int kTokTile = 16;         // tokens per tile, consecutive in batch order
constexpr int kTokMaxTokens = 512;   // largest max_tokens of this file's kernels
constexpr int kTokMaxOut = 256;      // largest max_loras * S * r (outputs of every adapter)
constexpr int kTokMaxLoraRank = 64;  // largest max_loras * r of the one-launch step
constexpr int kTokCols = 128;        // columns per expand chunk: 8 MFMA blocks of 16
constexpr int kTokRangeChunks = kShrinkWaves;  // chunks per expand unit, one per wave
// 16-token blocks per shrink tile (each wave holds them all, so an A piece
// feeds that many matrix-core ops and A is fetched once per 32 tokens)
constexpr int kTokShrinkMw = 1;
constexpr int kCounterInts = 64;     // ints per tile in the counter area (256 bytes)
constexpr int kConsumedAt = 32;      // the consumers' count sits 128 bytes after the arrivals'

// One chunk of a 16-token block of y in a lane: tokens 4*grp..4*grp+3, 8 columns each.
struct TokYBlock {
  u32x4 v[4];
};

struct TokenParams {
  const int32_t* mapping;
  int num_tokens;
  int max_tokens;
  int max_loras;
  int tiles;  // ceil(max_tokens / 16)
  // shrink
  const uint16_t* x;
  int64_t ldx;
  int hidden;
  const uint16_t* a[LORA_MAX_SLICES];
  int num_slices;
  int rank;
  int rank_shift;
  float scale;
  float* buf;
  uint32_t buf_bytes;
  int num_splits;
  int split_len;
  int num_groups;    // output groups of NB blocks over the nout outputs
  int nout;          // max_loras * S * r, ordered (adapter, slice, rank)
  int sr;            // S * r
  int shrink_tiles;  // shrink tiles of 16 * MW tokens: ceil(tiles / MW)
  int shrink_units;  // shrink_tiles * num_splits * num_groups
  int shrink_grid;   // workgroups of the shrink (a multiple of 8)
  // expand (one-launch step)
  const uint16_t* b[LORA_MAX_SLICES];
  int n[LORA_MAX_SLICES];
  int off[LORA_MAX_SLICES];
  int range_end[LORA_MAX_SLICES];  // running count of expand ranges through slice s
  int ranges;                      // expand units per tile
  uint16_t* y;
  int64_t ldy;
  int expand_units;  // tiles * ranges
  int expand_grid;   // workgroups of the expand (a multiple of 8)
  int* counters;     // [tiles][kCounterInts]
  int wait_polls;
  int start_delay_ticks;  // expand units' hold-off before their B loads, 100 MHz ticks
  int y_delay_ticks;      // ... before their y loads
  MetaOut meta_out;  // written by the workgroups past shrink_grid + expand_grid
};

// Unit of workgroup b among `grid` workgroups (a multiple of 8) serving `units`
// units, one each: each XCD (b % 8) takes one contiguous run of the unit
// order, so that the units that share operands (all tiles of one part and
// output group; all tiles of one column range) share that XCD's L2.  -1: none.
__device__ __forceinline__ int xcd_unit(int b, int units, int grid) {
  const int per = grid / kXcds;
  const int u = (b % kXcds) * per + b / kXcds;
  return u < units ? u : -1;
}

__device__ __forceinline__ int adapter_of(const TokenParams& p, int t) {
  const int tc = t < p.num_tokens ? t : p.num_tokens - 1;  // num_tokens >= 1 here
  const int32_t id = p.mapping[tc];
  return (t < p.num_tokens && id >= 0 && id < p.max_loras) ? id : -1;
}

// One shrink unit: part `part`, output group, tile m of MW * 16 tokens (MW
// 16-token blocks held by every wave, each A piece feeding MW matrix-core
// ops).  Every thread of the workgroup calls it.  COHERENT: the part is
// written with device-coherent stores (read by other workgroups of the same
// launch).  `red` is the unit's LDS: with one chunk per wave, each wave's
// A rows (16 * NB rows of 128 bytes, 2 KB per block) and then its share of the
// cross-wave sum, NB * 8 KB in all; otherwise the cross-wave sum, NB * 4 KB.
template <int NB, int MW, int DEPTH, bool COHERENT>
__device__ __forceinline__ void token_shrink_unit(const TokenParams& p, int u, f32x4* red,
                                                  const uint16_t* const* slice_a) {
  const int lane = lane_id();
  const int wave = wave_index();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int stiles = p.shrink_tiles;
  const int m = u % stiles;
  const int pg = u / stiles;
  const int part = pg / p.num_groups;
  const int o0 = (pg - part * p.num_groups) * 16 * NB;
  const int tbase = m * kTokTile * MW;
  if (tbase >= p.num_tokens) return;  // workgroup-uniform: no token of the batch

  // The map first (needed only at the store), then A and x, all unconditional.
  // Token of this lane's column (MFMA N index) in block mb: tbase + 16 mb + col.
  int lid[MW], tok[MW];
  const uint16_t* xrow[MW];
  uint32_t xmask[MW];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb) {
    tok[mb] = tbase + kTokTile * mb + col;
    lid[mb] = adapter_of(p, tok[mb]);
  }
  const int kbeg = part * p.split_len;
  const int kend = min(p.hidden, kbeg + p.split_len);

  // A rows: output o = o0 + 16*nb + col (MFMA M index); past the last: the last, masked.
  // (The row pointers serve the two-chunk register path; with one chunk per
  // wave A goes through LDS, addressed per 8-row group below.)
  const uint16_t* arow[NB];
  uint32_t amask[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int o = o0 + 16 * nb + col;
    const bool ok = o < p.nout;
    const int oc = ok ? o : p.nout - 1;
    const int l = oc / p.sr;
    const int rem = oc - l * p.sr;
    arow[nb] = slice_a[rem >> p.rank_shift] +
               (static_cast<int64_t>(l) * p.rank + (rem & (p.rank - 1))) * p.hidden;
    amask[nb] = opaque_mask(ok);
  }
#pragma unroll
  for (int mb = 0; mb < MW; ++mb) {
    const int tc = tok[mb] < p.num_tokens ? tok[mb] : p.num_tokens - 1;
    xrow[mb] = p.x + static_cast<int64_t>(tc) * p.ldx;
    xmask[mb] = opaque_mask(tok[mb] < p.num_tokens);
  }

  // The chunking of the grouped small-batch shrink (shrink.hip), element for
  // element: lane group g, MFMA i <-> elements [32i + 8g, +8) of a 64-element
  // chunk; wave w takes chunks w, w + 4, ... of the part; a chunk past the
  // part's end re-reads a piece inside the row and is masked.
  struct Chunk {
    u32x4 x[MW][2];
    u32x4 a[NB][2];
    uint32_t kmask[2];
  };
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
  auto load = [&](int kc, Chunk& c) {
    const bool full = kc + kShrinkChunk <= kend;  // wave-uniform
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = piece(kc, i, full, c.kmask[i]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) c.a[nb][i] = load16(arow[nb] + k);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t km;
      const int k = piece(kc, i, full, km);
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) c.x[mb][i] = load16(xrow[mb] + k);
    }
  };
  constexpr int kStride = kShrinkWaves * kShrinkChunk;
  int kc = kbeg + wave * kShrinkChunk;
  const int nw = kc < kend ? (kend - kc + kStride - 1) / kStride : 0;  // wave-uniform
  kc = kc < kend ? kc : ksafe;

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
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv[mb]), acc[mb][nb], 0,
              0, 0);
      }
    }
  };
  if constexpr (DEPTH == 1) {
    // At most one chunk per wave (parts of at most 256 elements).  x first,
    // into registers: read once (by this unit only), so with the streaming
    // hint, and ahead of A since x comes from HBM and A mostly from L2 (decode
    // step 9.96 -> 9.89 us for the hint, 9.20 -> 8.93 us for the order).
    u32x4 xv[MW][2];
    uint32_t kmask[2];
    {
      const bool full = kc + kShrinkChunk <= kend;  // wave-uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = piece(kc, i, full, kmask[i]);
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) xv[mb][i] = load16_stream(xrow[mb] + k);
      }
    }
    // A goes through this wave's own LDS region with whole-line loads:
    // instruction j fetches rows 8j..8j+7 of the group, 8 lanes per 128-byte
    // line (lane 8 rr + e reads row 8j + rr, piece e ^ rr, so the region holds
    // row R's piece q at 16-byte slot 8R + (q ^ (R & 7)) and the MFMA-layout
    // reads below hit distinct banks).  A load in the operand layout would
    // touch 16 lines for half a line each; whole lines move faster through
    // the CU.  Rows 8j..8j+7 are ranks 8i..8i+7 of one (adapter, slice) (r is
    // a multiple of 8): contiguous rows of one A_s.  A group past the last
    // output re-reads the last one (masked by amask).
    u32x4* const stg = reinterpret_cast<u32x4*>(red) + wave * (2 * NB * kWave);
    {
      const int rr = lane >> 3;
      const int kq = kc + 8 * ((lane & 7) ^ rr);
      const int lane_off = rr * p.hidden + (kq < kend ? kq : ksafe);
      int l = o0 / p.sr;  // (adapter, position in its S*r outputs) of row group j
      int rem = o0 - l * p.sr;
      // the slices' A from the kernel arguments, held as values in scalar
      // registers (an LDS read between these loads would wait for every one
      // issued before it; a select of argument addresses, for a scalar load)
      uint64_t sa_v[LORA_MAX_SLICES];
#pragma unroll
      for (int s = 0; s < LORA_MAX_SLICES; ++s) {
        sa_v[s] = reinterpret_cast<uint64_t>(p.a[s]);
        asm volatile("" : "+s"(sa_v[s]));
      }
#pragma unroll
      for (int j = 0; j < 2 * NB; ++j) {
        const bool past = o0 + 8 * j >= p.nout;  // workgroup-uniform
        const int lj = past ? p.max_loras - 1 : l;
        const int rj = past ? p.sr - 8 : rem;
        const int sj = rj >> p.rank_shift;
        uint64_t sa = sa_v[0];
#pragma unroll
        for (int s = 1; s < LORA_MAX_SLICES; ++s) sa = sj == s ? sa_v[s] : sa;
        const uint16_t* base = reinterpret_cast<const uint16_t*>(sa) +
                               (static_cast<int64_t>(lj) * p.rank + (rj & (p.rank - 1))) * p.hidden;
        load16_to_lds(base + lane_off, stg + j * kWave);
        rem += 8;
        if (rem == p.sr) {
          rem = 0;
          ++l;
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (nw > 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int mb = 0; mb < MW; ++mb) xv[mb][i] &= xmask[mb] & kmask[i];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 av = stg[(16 * nb + col) * 8 + ((4 * i + grp) ^ (col & 7))] & amask[nb];
#pragma unroll
          for (int mb = 0; mb < MW; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv[mb][i]),
                acc[mb][nb], 0, 0, 0);
        }
      }
    }
  } else if (nw > 0) {
    // two chunks in flight, alternating two register sets (as in shrink.hip)
    Chunk c0, c1;
    load(kc, c0);
    int j = 0;
    for (; j + 2 < nw; j += 2) {
      load(kc + (j + 1) * kStride, c1);
      __builtin_amdgcn_sched_barrier(0);
      mma(c0);
      load(kc + (j + 2) * kStride, c0);
      __builtin_amdgcn_sched_barrier(0);
      mma(c1);
    }
    if (j + 1 < nw) {
      load(kc + (j + 1) * kStride, c1);
      __builtin_amdgcn_sched_barrier(0);
      mma(c0);
      mma(c1);
    } else {
      mma(c0);
    }
  }

  // The four waves' sums in wave order, one 16-token block at a time; wave w
  // stores output blocks w, w+4, ...  This lane holds outputs o0 + 16*nb +
  // 4*grp + j (j < 4) of token tok[mb]: one adapter and one slice (r is a
  // multiple of 8); kept if the adapter is the token's.  Each wave's sums go
  // to the start of its own A region (with one chunk per wave), which only it
  // has read so far.
  constexpr int kRedWave = DEPTH == 1 ? 2 * NB : NB;  // f32x4 blocks of 64 between waves
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.buf, p.buf_bytes);
#pragma unroll
  for (int mb = 0; mb < MW; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(wave * kRedWave + nb) * kWave + lane] = acc[mb][nb];
    __syncthreads();
    for (int nb = wave; nb < NB; nb += kShrinkWaves) {
      f32x4 v = red[nb * kWave + lane];
#pragma unroll
      for (int w = 1; w < kShrinkWaves; ++w) v += red[(w * kRedWave + nb) * kWave + lane];
      const int o = o0 + 16 * nb + 4 * grp;
      const int l = o / p.sr;
      if (o < p.nout && l == lid[mb]) {
        const int rem = o - l * p.sr;
        const int s = rem >> p.rank_shift;
        v *= p.scale;
        const int64_t e =
            ((static_cast<int64_t>(part) * p.num_slices + s) * p.max_tokens + tok[mb]) * p.rank +
            (rem & (p.rank - 1));
        if constexpr (COHERENT) {
          store16_coherent(rb, static_cast<uint32_t>(e * 4), __builtin_bit_cast(u32x4, v));
        } else {
          store16(p.buf + e, __builtin_bit_cast(u32x4, v));
        }
      }
    }
    __syncthreads();  // red is reused by the next block (or the caller's next unit)
  }
}

// B chunk of one adapter (128 rows of RANK bf16) in a wave's LDS region: the
// XOR-swizzled layout of expand.hip (bslot), one region per adapter slot.
template <int RANK>
__device__ __forceinline__ int tok_bslot(int row, int pr) {
  if constexpr (RANK == 8) return row ^ ((row >> 4) & 7);
  return (row * (RANK / 8) + pr) ^ ((row >> 3) & 15);
}

// One expand unit of the one-launch step: tile m, slice s, range of 4 chunks
// (wave w takes chunk w of the range).  LCAP >= max_loras.
template <int RANK, int NB, int MW, int DEPTH, int LCAP, bool WT>
__device__ __forceinline__ void token_expand_unit(const TokenParams& p, int u, u32x4* lds,
                                                  const uint16_t* const* slice_a, int* flag) {
  constexpr int kRegion = 16 * RANK;        // u32x4 per adapter chunk
  constexpr int kPieces = RANK / 4;         // 16-byte pieces per lane per adapter chunk
  constexpr int kRowPieces = RANK / 8;
  constexpr int kPer = RANK == 8 ? 4 : 8;   // ranks of the rank operand per lane
  const int lane = lane_id();
  const int wave = wave_index();
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int khalf = grp & 1;
  const bool use_lo = grp >= 2;
  const int m = u % p.tiles;
  const int gr = u / p.tiles;
  int* const ctr = p.counters + m * kCounterInts;
  const int target = p.num_splits * p.num_groups;
  const int t0 = m * kTokTile;

  int consumed_before = 0;
  bool live = t0 < p.num_tokens;  // workgroup-uniform
  if (live) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < LORA_MAX_SLICES - 1; ++i)
      s += (i < p.num_slices - 1 && gr >= p.range_end[i]) ? 1 : 0;
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
    const int chunks_s = (n_s + kTokCols - 1) / kTokCols;
    const int ch = (gr - r_before) * kTokRangeChunks + wave;
    const bool has_chunk = ch < chunks_s;
    const int chc = has_chunk ? ch : chunks_s - 1;

    // First round trip: the ids (y and B follow after their hold-offs).
    const int ta = t0 + c;  // rank-operand row
    const int la = adapter_of(p, ta);
    int td[4], ld[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      td[j] = t0 + 4 * grp + j;
      ld[j] = adapter_of(p, td[j]);
    }
    u32x4 bv[LCAP][kPieces];
    auto load_b = [&]() {
#pragma unroll
      for (int l = 0; l < LCAP; ++l) {
        const int lc = l < p.max_loras ? l : p.max_loras - 1;
        const uint16_t* bmat = bslice + static_cast<int64_t>(lc) * n_s * RANK;
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
          const int q = lane + kWave * i;
          const int row = chc * kTokCols + q / kRowPieces;
          const int rowc = row < n_s ? row : n_s - 1;
          bv[l][i] = load16(bmat + static_cast<int64_t>(rowc) * RANK + 8 * (q % kRowPieces));
        }
      }
    };
    int64_t yrow[4];
    bool dval[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dval[j] = ld[j] >= 0;
      yrow[j] = static_cast<int64_t>(dval[j] ? td[j] : t0) * p.ldy + off_s;
    }
    const int ycol = chc * kTokCols + 8 * c;
    const int ycolc = ycol < n_s ? ycol : n_s - 8;
    TokYBlock yb;
    auto load_y = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j) yb.v[j] = load16_stream(p.y + yrow[j] + ycolc);
    };
    // Hold this unit's y and B loads back while the shrink units' loads are
    // served: they share each CU's fetch path with them, and the parts the
    // unit waits for come sooner that way; y and B still arrive before the
    // parts do.  y (from HBM, the slower to arrive) goes out first, after a
    // shorter hold-off, B (mostly L2 hits) after the longer one: on the decode
    // batch 9.23 us per step against 9.90 with both at 2 us (8.7 us once the
    // shrink's x went out ahead of its A).  Timed on the chip's constant
    // 100 MHz clock from here.
    {
      const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
      auto hold_until = [&](int ticks) {
        while (__builtin_amdgcn_s_memrealtime() - t_start < static_cast<uint64_t>(ticks))
          __builtin_amdgcn_s_sleep(2);
        asm volatile("" ::: "memory");
      };
      hold_until(p.y_delay_ticks);
      load_y();
      hold_until(p.start_delay_ticks);
      load_b();
    }

    // Every adapter's chunk into this wave's own LDS regions, while the
    // parts are still being computed.
    u32x4* const bw = lds + wave * LCAP * kRegion;
    auto stage_b = [&]() {
#pragma unroll
      for (int l = 0; l < LCAP; ++l)
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
          const int q = lane + kWave * i;
          bw[l * kRegion + tok_bslot<RANK>(q / kRowPieces, q % kRowPieces)] = bv[l][i];
        }
    };
    stage_b();

    // The tile's adapters (every wave holds the same 16 rows in lanes c).
    const bool any = __ballot(la >= 0) != 0;  // workgroup-uniform
    bool ready = true;
    if (any) {
      if (wave == 0) {
        // Four polls in flight, issued a short sleep apart, each checked as it
        // returns (loads return in order) and reissued: a count that becomes
        // complete is seen about one round trip later, not up to two.
        bool done = false;
        if (!done && p.wait_polls > 0) {
          auto poll = [&]() {
            __builtin_amdgcn_s_sleep(2);
            return __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          };
          int v0 = poll(), v1 = poll(), v2 = poll(), v3 = poll();
          for (int polls = 4; polls < p.wait_polls + 4; polls += 4) {
            if (v0 >= target) { done = true; break; }
            v0 = poll();
            if (v1 >= target) { done = true; break; }
            v1 = poll();
            if (v2 >= target) { done = true; break; }
            v2 = poll();
            if (v3 >= target) { done = true; break; }
            v3 = poll();
          }
        }
        if (lane == 0) *flag = done ? 1 : 0;
      }
      __syncthreads();
      ready = *flag != 0;
    }
    if (any) {
      if (!ready) {
        // Out of polls: compute every part of this tile here (the shrink
        // units' code, so the same bits, over the LDS the B chunks were
        // staged in), then fetch and stage B again and fetch y again (their
        // registers are free during the shrink).
        __syncthreads();  // every wave has read *flag
        for (int pg = 0; pg < target; ++pg)
          token_shrink_unit<NB, MW, DEPTH, true>(p, pg * p.shrink_tiles + m / MW,
                                                 reinterpret_cast<f32x4*>(lds), slice_a);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_b();
        load_y();
        stage_b();
      }
      asm volatile("" ::: "memory");  // the parts are read after the wait

      // Rank vectors of the tile's 16 rows for slice s, summed over the parts
      // in part order, by wave 0 alone (lane L: row L / 4, ranks RANK/4 * (L % 4)
      // onwards: every part element is loaded once) into LDS; then each lane
      // takes row c's ranks [k0, k0 + kPer) and splits them hi/lo (lane groups
      // 0-1 hi, 2-3 lo); zero on the steps of other adapters.
      float* const rsum = reinterpret_cast<float*>(lds + kShrinkWaves * LCAP * kRegion);
      if (wave == 0) {
        constexpr int kEach = RANK / 4;  // ranks per lane: 2 or 4
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.buf, p.buf_bytes);
        const int row = lane >> 2;
        const int kk = kEach * (lane & 3);
        const int tr = t0 + row < p.num_tokens ? t0 + row : t0;
        const int64_t plane = static_cast<int64_t>(p.num_slices) * p.max_tokens * RANK;
        const int64_t e0 = (static_cast<int64_t>(s) * p.max_tokens + tr) * RANK + kk;
        float v[kEach];
#pragma unroll
        for (int e = 0; e < kEach; ++e) v[e] = 0.f;
        constexpr int kGroup = 16;
        for (int sp0 = 0; sp0 < p.num_splits; sp0 += kGroup) {
          uint32_t w[kGroup][kEach];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const int sp = sp0 + i < p.num_splits ? sp0 + i : sp0;
            const uint32_t off = static_cast<uint32_t>((e0 + sp * plane) * 4);
            if constexpr (kEach == 2) {
              const u32x2 q = load8_coherent(rb, off);
              w[i][0] = q[0];
              w[i][1] = q[1];
            } else {
              const u32x4 q = load16_coherent(rb, off);
#pragma unroll
              for (int e = 0; e < 4; ++e) w[i][e] = q[e];
            }
          }
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const uint32_t pm = opaque_mask(sp0 + i < p.num_splits);
#pragma unroll
            for (int e = 0; e < kEach; ++e) v[e] += __uint_as_float(w[i][e] & pm);
          }
        }
#pragma unroll
        for (int e = 0; e < kEach; ++e) rsum[row * RANK + kk + e] = v[e];
      }
      __syncthreads();
      const int k0 = kPer * khalf;
      float v[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[e] = rsum[c * RANK + k0 + e];
      uint32_t words[kPer / 2];
#pragma unroll
      for (int e = 0; e < kPer; e += 2) {
        const uint32_t hi = pack_bf16x2(v[e], v[e + 1]);
        words[e / 2] = use_lo ? pack_bf16x2(v[e] - bf16_lo(hi), v[e + 1] - bf16_hi(hi)) : hi;
      }

      // acc = y + sum over the tile's adapters of (row mask) buf . B_l^T
      f32x4 acc[8];
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t wv = yb.v[j][b >> 1];
          acc[b][j] = (b & 1) ? bf16_hi(wv) : bf16_lo(wv);
        }
      // Every adapter slot, straight-line code (no branch, so the LDS reads of
      // one slot go out while the previous slot's MFMAs run): the rank operand
      // is zero on the rows of other adapters, and a slot past max_loras holds
      // a copy of the last slot's chunk and meets only zero rows.
#pragma unroll
      for (int l = 0; l < LCAP; ++l) {
        const uint32_t km = opaque_mask(la == l);
        const u32x4* rl = bw + l * kRegion;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          if constexpr (RANK == 8) {
            const u32x2 op = {words[0] & km, words[1] & km};
            const u32x2 bb = reinterpret_cast<const u32x2*>(rl + tok_bslot<RANK>(8 * c + b, 0))[khalf];
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(i16x4, op), __builtin_bit_cast(i16x4, bb), acc[b], 0, 0, 0);
          } else {
            const u32x4 op = {words[0] & km, words[1] & km, words[2] & km, words[3] & km};
            const u32x4 bb = rl[tok_bslot<RANK>(8 * c + b, khalf)];
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, op), __builtin_bit_cast(bf16x8, bb), acc[b], 0, 0, 0);
          }
        }
      }
      // WT: y goes out written through to the level every XCD shares (with
      // the streaming hint), so the launch ends without dirty y lines in the
      // XCDs' L2s to write back (decode batch: 10.26 -> 10.0 us per step).  Its
      // byte offsets are 32-bit, so the host picks WT only where y spans less
      // than 4 GiB.  (The extent comes from arguments already there: a new
      // field shifts the others, and where they sit in the argument block
      // measurably costs time here.)
      const bool col_ok = has_chunk && ycol < n_s;
      const __amdgpu_buffer_rsrc_t yr =
          buffer_rsrc(p.y, static_cast<uint32_t>(static_cast<int64_t>(p.num_tokens) * p.ldy * 2));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (col_ok && dval[j]) {
          const u32x4 out = {pack_bf16x2(acc[0][j], acc[1][j]), pack_bf16x2(acc[2][j], acc[3][j]),
                             pack_bf16x2(acc[4][j], acc[5][j]), pack_bf16x2(acc[6][j], acc[7][j])};
          if constexpr (WT) {
            store16_stream_coherent(yr, static_cast<uint32_t>((yrow[j] + ycol) * 2), out);
          } else {
            store16_stream(p.y + yrow[j] + ycol, out);
          }
        }
      }
    }
  }
  // Count this unit out (after its wait, and after its stores have been
  // issued, so the atomic's round trip overlaps their drain); the tile's last
  // consumer returns both counters to zero (a part that arrives after it,
  // possible only after a bounded wait ran out, brings the arrivals back up
  // to zero).
  if (threadIdx.x == 0)
    consumed_before = __hip_atomic_fetch_add(ctr + kConsumedAt, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0 && consumed_before == p.ranges - 1) {
    __hip_atomic_fetch_add(ctr, -target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(ctr + kConsumedAt, -p.ranges, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// STEP = false: lora_prepare_and_shrink for small batches (shrink workgroups,
// then metadata workgroups; plain stores, no counters).  STEP = true: the
// one-launch step.  Dynamic LDS: the shrink's (NB * 8 KB with one chunk per
// wave, NB * 4 KB otherwise), the expand's B regions (4 waves * LCAP
// adapters * 256 * RANK bytes) or the metadata's, whichever is largest: every
// workgroup does one kind of work, so they share it.
// Waves per SIMD each instantiation is built for: three where the registers
// fit without spilling (the decode shapes), so that a one-launch grid of
// shrink, expand and metadata workgroups is resident at once; two otherwise.
template <int NB, int DEPTH>
constexpr int token_waves() {
  return NB <= (DEPTH == 1 ? 6 : 2) ? 3 : 2;
}

template <int NB, int MW, int DEPTH, int RANK, int LCAP, bool STEP, bool WT = false>
__global__ __launch_bounds__(kShrinkThreads)
__attribute__((amdgpu_waves_per_eu(token_waves<NB, DEPTH>())))
void token_kernel(TokenParams p) {
  extern __shared__ u32x4 tok_lds[];
  __shared__ const uint16_t* slice_a[LORA_MAX_SLICES];
  __shared__ int flag;
  const int b = blockIdx.x;
  const int work = p.shrink_grid + (STEP ? p.expand_grid : 0);
  if (b >= work) {  // workgroup-uniform
    metadata_group<kShrinkThreads>(p.mapping, p.num_tokens, p.max_loras, p.meta_out, b - work,
                                   *reinterpret_cast<MetaLds<kShrinkThreads>*>(tok_lds));
    return;
  }
  if (threadIdx.x < LORA_MAX_SLICES) slice_a[threadIdx.x] = p.a[threadIdx.x];
  __syncthreads();
  if (b < p.shrink_grid) {
    const int u = xcd_unit(b, p.shrink_units, p.shrink_grid);
    if (u < 0) return;
    token_shrink_unit<NB, MW, DEPTH, STEP>(p, u, reinterpret_cast<f32x4*>(tok_lds), slice_a);
    if constexpr (STEP) {
      // the part is complete at the level every XCD reads from: count it in,
      // in each 16-token tile the unit covers
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int m0 = (u % p.shrink_tiles) * MW;
      if (threadIdx.x < MW && m0 + static_cast<int>(threadIdx.x) < p.tiles)
        __hip_atomic_fetch_add(p.counters + (m0 + threadIdx.x) * kCounterInts, 1,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if constexpr (STEP) {
    const int u = xcd_unit(b - p.shrink_grid, p.expand_units, p.expand_grid);
    if (u >= 0) token_expand_unit<RANK, NB, MW, DEPTH, LCAP, WT>(p, u, tok_lds, slice_a, &flag);
  }
}

// ------------------------------------------------------------------ host --

// Whether every wave has at most one 64-element chunk of a part (parts of at
// most 4 * 64 elements): then one chunk register set, else two.
static bool token_one_chunk(int split_len) { return split_len <= kShrinkWaves * kShrinkChunk; }

// Output blocks per group and groups over nout outputs: blocks of 16, at most
// 8 per group (6 with two chunk register sets, which would spill at 8), the
// block count per group rounded up to 2, 4, 6 or 8.
static void token_groups(int nout, bool one_chunk, int& nb, int& groups) {
  const int total = (nout + 15) / 16;
  const int cap = one_chunk ? 8 : 6;
  groups = (total + cap - 1) / cap;
  int per = (total + groups - 1) / groups;
  nb = per <= 2 ? 2 : per <= 4 ? 4 : per <= 6 ? 6 : 8;
}

bool token_shrink_fits(int max_tokens, int max_loras, int num_slices, int rank) {
  return max_tokens <= kTokMaxTokens &&
         static_cast<int64_t>(max_loras) * num_slices * rank <= kTokMaxOut;
}

bool token_step_fits(int max_tokens, int max_loras, int num_slices, int rank) {
  return token_shrink_fits(max_tokens, max_loras, num_slices, rank) &&
         (rank == 8 || rank == 16) && max_loras * rank <= kTokMaxLoraRank;
}

// Counters of lora_fused_step_static: a file-scope device array in place of
// the caller's workspace, for callers that cannot allocate.  It covers the
// largest one-launch batch (512 token slots, 32 tiles: 8 KB); every GPU the
// library runs on holds its own copy until the process ends, zero-filled when
// the code object is loaded, and every call leaves the counters it used at
// zero again.  In host code `scratch` names a host-side stand-in, never the
// device address: that comes from hipGetSymbolAddress, once per device.
constexpr int kScratchTiles = kTokMaxTokens / kTokTile;
static __device__ __align__(256) int scratch[kScratchTiles * kCounterInts];

constexpr int kScratchDevices = 64;
static int* g_scratch_ptr[kScratchDevices];
static std::mutex g_scratch_mu;

int64_t token_step_scratch_bytes() { return static_cast<int64_t>(sizeof(scratch)); }

// Device address of this device's copy of `scratch` (the current device's:
// the one the caller's stream belongs to).  Resolved on the first call on each
// device, with that device current.
hipError_t token_step_scratch(int** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<int*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int64_t token_step_workspace_bytes(int max_tokens) {
  const int64_t tiles = (static_cast<int64_t>(max_tokens) + kTokTile - 1) / kTokTile;
  return tiles * kCounterInts * static_cast<int64_t>(sizeof(int));
}

static TokenParams token_params(const int32_t* mapping, int num_tokens, const uint16_t* x,
                                int64_t ldx, int hidden, const uint16_t* const* lora_a,
                                int num_slices, int rank, float scale, float* buf,
                                int num_splits, const lora_meta_t& meta, int max_tokens,
                                int max_loras, int& nb) {
  TokenParams p{};
  p.mapping = mapping;
  p.num_tokens = num_tokens;
  p.max_tokens = max_tokens;
  p.max_loras = max_loras;
  p.tiles = (max_tokens + kTokTile - 1) / kTokTile;
  p.x = x;
  p.ldx = ldx;
  p.hidden = hidden;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) p.a[s] = s < num_slices ? lora_a[s] : lora_a[0];
  p.num_slices = num_slices;
  p.rank = rank;
  p.rank_shift = rank == 8 ? 3 : rank == 16 ? 4 : rank == 32 ? 5 : 6;
  p.scale = scale;
  p.buf = buf;
  p.buf_bytes = static_cast<uint32_t>(static_cast<int64_t>(num_splits) * num_slices * max_tokens *
                                      rank * 4);
  p.num_splits = num_splits;
  p.split_len = shrink_split_len(hidden, num_splits);
  p.nout = max_loras * num_slices * rank;
  p.sr = num_slices * rank;
  int groups = 1;
  token_groups(p.nout, token_one_chunk(p.split_len), nb, groups);
  p.num_groups = groups;
  p.shrink_tiles = (p.tiles + kTokShrinkMw - 1) / kTokShrinkMw;
  p.shrink_units = p.shrink_tiles * num_splits * groups;
  p.shrink_grid = (p.shrink_units + kXcds - 1) / kXcds * kXcds;
  p.meta_out = MetaOut{meta.sorted_token_ids, meta.active_lora_ids, meta.num_tokens_per_lora,
                       meta.lora_token_start, meta.num_active, meta.tile_token_ids,
                       meta.tile_lora, meta.num_tiles, meta.num_runs};
  return p;
}

// Default hold-offs of the expand units (ns), in proportion to what a shrink
// unit loads (A and x): B after 43 ns per KB, y after 11 (measured on the
// decode batch, a unit reading 56 KB: best at B 2.2-2.4 us with y 0.6-0.8 us;
// both at 2 us cost 7%, y at 0 or 1.2 us, or B at 2.0 or 2.8 us, 2-10%).
static int64_t token_shrink_unit_kb(const TokenParams& p, int nb) {
  return static_cast<int64_t>(16 * nb + kTokTile * kTokShrinkMw) * p.split_len * 2 / 1024;
}
static int token_step_default_delay_ns(const TokenParams& p, int nb) {
  return static_cast<int>(43 * token_shrink_unit_kb(p, nb));
}
static int token_step_default_y_delay_ns(const TokenParams& p, int nb) {
  return static_cast<int>(11 * token_shrink_unit_kb(p, nb));
}

template <int NB, int DEPTH, int RANK, int LCAP, bool STEP, bool WT>
static hipError_t launch_token(const TokenParams& params, hipStream_t stream) {
  constexpr int MW = kTokShrinkMw;
  TokenParams p = params;
  const int grid = p.shrink_grid + (STEP ? p.expand_grid : 0) + p.max_loras + 1;
  // one chunk per wave: A staged per wave (twice the sums' size), the sums in it
  const size_t red = static_cast<size_t>(kShrinkWaves) * NB * kWave * sizeof(f32x4) * (DEPTH == 1 ? 2 : 1);
  const size_t bst = STEP ? static_cast<size_t>(kShrinkWaves) * LCAP * 16 * RANK * sizeof(u32x4) +
                               16 * RANK * sizeof(float)
                          : 0;
  size_t lds = red > bst ? red : bst;
  lds = lds > sizeof(MetaLds<kShrinkThreads>) ? lds : sizeof(MetaLds<kShrinkThreads>);
  if constexpr (STEP) {
    // Default hold-offs (negative ticks): none when the shrink's workgroups
    // alone fill every slot of the device, since the expand's then start only
    // as shrink workgroups end, with nothing left to make way for (rank 16,
    // 256 tokens, two workgroups per CU: 14.1 -> 12.9 us); else the sizes'
    // defaults.  Workgroups per CU: looked up once per kernel and kept.
    if (p.start_delay_ticks < 0 || p.y_delay_ticks < 0) {
      static const int per_cu = [lds] {
        int v = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &v, token_kernel<NB, MW, DEPTH, RANK, LCAP, STEP, WT>, kShrinkThreads, lds) ==
                       hipSuccess
                   ? v
                   : 0;
      }();
      const bool crowded = per_cu > 0 && p.shrink_grid >= per_cu * kCus;
      if (p.start_delay_ticks < 0)
        p.start_delay_ticks = crowded ? 0 : (token_step_default_delay_ns(p, NB) + 5) / 10;
      if (p.y_delay_ticks < 0)
        p.y_delay_ticks = crowded ? 0 : (token_step_default_y_delay_ns(p, NB) + 5) / 10;
    }
  }
  hipLaunchKernelGGL((token_kernel<NB, MW, DEPTH, RANK, LCAP, STEP, WT>), dim3(grid), dim3(kShrinkThreads),
                     lds, stream, p);
  return hipGetLastError();
}

template <int RANK, int LCAP, bool STEP, bool WT = false>
static hipError_t launch_token_nb(const TokenParams& p, int nb, hipStream_t stream) {
  if (token_one_chunk(p.split_len)) {
    switch (nb) {
      case 2: return launch_token<2, 1, RANK, LCAP, STEP, WT>(p, stream);
      case 4: return launch_token<4, 1, RANK, LCAP, STEP, WT>(p, stream);
      case 6: return launch_token<6, 1, RANK, LCAP, STEP, WT>(p, stream);
      default: return launch_token<8, 1, RANK, LCAP, STEP, WT>(p, stream);
    }
  }
  switch (nb) {  // at most 6 (token_groups)
    case 2: return launch_token<2, 2, RANK, LCAP, STEP, WT>(p, stream);
    case 4: return launch_token<4, 2, RANK, LCAP, STEP, WT>(p, stream);
    default: return launch_token<6, 2, RANK, LCAP, STEP, WT>(p, stream);
  }
}

// lora_prepare_and_shrink on a small batch: one launch, the shrink in batch
// order beside the metadata workgroups.  The caller checked token_shrink_fits.
hipError_t launch_token_prep_shrink(const int32_t* mapping, int num_tokens, const uint16_t* x,
                                    int64_t ldx, int hidden, const uint16_t* const* lora_a,
                                    int num_slices, int rank, float scale, float* buf,
                                    int num_splits, const lora_meta_t& meta, int max_tokens,
                                    int max_loras, hipStream_t stream) {
  int nb = 2;
  const TokenParams p = token_params(mapping, num_tokens, x, ldx, hidden, lora_a, num_slices, rank,
                                     scale, buf, num_splits, meta, max_tokens, max_loras, nb);
  return launch_token_nb<8, 4, false>(p, nb, stream);
}


// The one-launch step.  The caller checked token_step_fits and the workspace.
hipError_t launch_token_step(const int32_t* mapping, int num_tokens, const uint16_t* x,
                             int64_t ldx, int hidden, const uint16_t* const* lora_a,
                             const uint16_t* const* lora_b, const int32_t* slice_sizes,
                             int num_slices, int rank, float scale, float* buf, int num_splits,
                             uint16_t* y, int64_t ldy, const lora_meta_t& meta, int* counters,
                             int wait_polls, int start_delay_ns, int y_delay_ns, int max_tokens,
                             int max_loras, hipStream_t stream) {
  int nb = 2;
  TokenParams p = token_params(mapping, num_tokens, x, ldx, hidden, lora_a, num_slices, rank,
                               scale, buf, num_splits, meta, max_tokens, max_loras, nb);
  int ranges = 0, off = 0;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) {
    if (s < num_slices) {
      p.b[s] = lora_b[s];
      p.n[s] = slice_sizes[s];
      p.off[s] = off;
      off += slice_sizes[s];
      const int chunks = (slice_sizes[s] + kTokCols - 1) / kTokCols;
      ranges += (chunks + kTokRangeChunks - 1) / kTokRangeChunks;
    } else {
      p.b[s] = lora_b[0];
      p.n[s] = 0;
      p.off[s] = off;
    }
    p.range_end[s] = ranges;
  }
  p.ranges = ranges;
  p.y = y;
  p.ldy = ldy;
  p.expand_units = p.tiles * ranges;
  p.expand_grid = (p.expand_units + kXcds - 1) / kXcds * kXcds;
  p.counters = counters;
  p.wait_polls = wait_polls;
  // negative: the defaults, resolved at the launch (they depend on the kernel)
  p.start_delay_ticks = start_delay_ns < 0 ? -1 : (start_delay_ns + 5) / 10;
  p.y_delay_ticks = y_delay_ns < 0 ? -1 : (y_delay_ns + 5) / 10;
  // y written through where its byte offsets fit 32 bits (all but y of 4 GiB
  // or more)
  const bool wt = static_cast<int64_t>(num_tokens) * ldy * 2 < (int64_t{1} << 32);
  if (rank == 8) {
    if (max_loras <= 4)
      return wt ? launch_token_nb<8, 4, true, true>(p, nb, stream)
                : launch_token_nb<8, 4, true, false>(p, nb, stream);
    return wt ? launch_token_nb<8, 8, true, true>(p, nb, stream)
              : launch_token_nb<8, 8, true, false>(p, nb, stream);
  }
  return wt ? launch_token_nb<16, 4, true, true>(p, nb, stream)
            : launch_token_nb<16, 4, true, false>(p, nb, stream);
}

}  // namespace lora
