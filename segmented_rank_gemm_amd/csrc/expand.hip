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
constexpr int kExpandTile = 16;    // tokens per wave unit (the MFMA M dimension)
constexpr int kExpandCols = 128;   // columns per chunk: 8 MFMA blocks of 16

struct ExpandParams {
  const float* buf;
  int num_splits;
  const uint16_t* b[LORA_MAX_SLICES];
  int n[LORA_MAX_SLICES];
  int off[LORA_MAX_SLICES];
  int range_end[LORA_MAX_SLICES];  // running count of column ranges through slice s
  int num_slices;
  int chunks_per_range;
  uint16_t* y;
  int64_t ldy;
  const int32_t* sorted;
  const int32_t* active_ids;
  const int32_t* counts;
  const int32_t* starts;
  const int32_t* num_active;
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

template <int RANK>
__global__ __launch_bounds__(kExpandThreads) void expand_kernel(ExpandParams p) {
  __shared__ SegmentTable tab;
  build_segment_table<kExpandTile>(tab, p.active_ids, p.counts, p.starts, p.num_active,
                                   p.max_loras, p.max_tokens);
  const int num_tiles = tab.num_tiles;
  const int ranges = p.range_end[p.num_slices - 1];
  const int units = num_tiles * ranges;

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int c = lane & 15;   // MFMA row (token) for the buf operand, column for B / D
  const int grp = lane >> 4;
  const int khalf = grp & 1;  // which half of each 16-rank (or 8-rank) group
  const bool use_lo = grp >= 2;

  for (int u = blockIdx.x * kExpandWaves + wave; u < units; u += gridDim.x * kExpandWaves) {
    const int m = u % num_tiles;
    const int cr = u / num_tiles;
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
    const int chunk_begin = (cr - r_before) * p.chunks_per_range;
    const int chunks_s = (n_s + kExpandCols - 1) / kExpandCols;
    const int chunk_end = min(chunks_s, chunk_begin + p.chunks_per_range);

    const Tile tile = resolve_tile<kExpandTile>(tab, m);

    // Rank operand: token c of the tile, fp32 sum over the shrink's parts.
    RankOperand<RANK> a;
    {
      const int ta = c < tile.rows ? token_at(p.sorted, tile.first + c, p.max_tokens) : -1;
      constexpr int kPer = RANK == 8 ? 4 : 8;  // ranks per lane per MFMA
#pragma unroll
      for (int q = 0; q < RankOperand<RANK>::kSteps; ++q) {
        float v[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) v[e] = 0.f;
        if (ta >= 0) {
          const int k0 = RANK == 8 ? 4 * khalf : 16 * q + 8 * khalf;
          for (int sp = 0; sp < p.num_splits; ++sp) {
            const float* src = p.buf + ((static_cast<int64_t>(sp) * p.num_slices + s) * p.max_tokens + ta) *
                                           RANK + k0;
#pragma unroll
            for (int e4 = 0; e4 < kPer; e4 += 4) {
              const f32x4 w = __builtin_bit_cast(f32x4, load16(src + e4));
              v[e4 + 0] += w[0];
              v[e4 + 1] += w[1];
              v[e4 + 2] += w[2];
              v[e4 + 3] += w[3];
            }
          }
        }
        uint32_t packed[kPer / 2];
#pragma unroll
        for (int e = 0; e < kPer; e += 2) {
          const uint32_t hi = pack_bf16x2(v[e], v[e + 1]);
          if (use_lo) {
            packed[e / 2] = pack_bf16x2(v[e] - bf16_lo(hi), v[e + 1] - bf16_hi(hi));
          } else {
            packed[e / 2] = hi;
          }
        }
        if constexpr (RANK == 8) {
          a.op[q] = __builtin_bit_cast(i16x4, u32x2{packed[0], packed[1]});
        } else {
          a.op[q] = __builtin_bit_cast(bf16x8, u32x4{packed[0], packed[1], packed[2], packed[3]});
        }
      }
    }

    // Output tokens of this lane in the D layout: rows 4*grp + j.
    int td[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * grp + j;
      td[j] = r < tile.rows ? token_at(p.sorted, tile.first + r, p.max_tokens) : -1;
    }
    const uint16_t* bmat = bslice + static_cast<int64_t>(tile.lora) * n_s * RANK;

    for (int ch = chunk_begin; ch < chunk_end; ++ch) {
      const int col = ch * kExpandCols + 8 * c;  // first of this lane's 8 columns
      const bool col_ok = col < n_s;             // n_s is a multiple of 8

      u32x4 yv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        yv[j] = (col_ok && td[j] >= 0)
                    ? load16(p.y + static_cast<int64_t>(td[j]) * p.ldy + off_s + col)
                    : u32x4{0u, 0u, 0u, 0u};
      }

      f32x4 acc[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = yv[j][b >> 1];
          acc[b][j] = (b & 1) ? bf16_hi(w) : bf16_lo(w);
        }
      }

#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint16_t* brow = bmat + static_cast<int64_t>(col + b) * RANK;
#pragma unroll
        for (int q = 0; q < RankOperand<RANK>::kSteps; ++q) {
          if constexpr (RANK == 8) {
            const u32x2 bw = col_ok ? load8(brow + 4 * khalf) : u32x2{0u, 0u};
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                a.op[q], __builtin_bit_cast(i16x4, bw), acc[b], 0, 0, 0);
          } else {
            const u32x4 bw = col_ok ? load16(brow + 16 * q + 8 * khalf) : u32x4{0u, 0u, 0u, 0u};
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a.op[q], __builtin_bit_cast(bf16x8, bw), acc[b], 0, 0, 0);
          }
        }
      }

#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (col_ok && td[j] >= 0) {
          const u32x4 out = {pack_bf16x2(acc[0][j], acc[1][j]), pack_bf16x2(acc[2][j], acc[3][j]),
                             pack_bf16x2(acc[4][j], acc[5][j]), pack_bf16x2(acc[6][j], acc[7][j])};
          store16(p.y + static_cast<int64_t>(td[j]) * p.ldy + off_s + col, out);
        }
      }
    }
  }
}

template <int RANK>
hipError_t launch_expand_rank(const ExpandParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(expand_kernel<RANK>, dim3(grid), dim3(kExpandThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_expand(const float* buf, int num_splits, const uint16_t* const* lora_b,
                         const int32_t* slice_sizes, int num_slices, int rank, uint16_t* y,
                         int64_t ldy, const lora_meta_t& meta, int max_tokens, int max_loras,
                         int num_cus, hipStream_t stream) {
  ExpandParams p{};
  p.buf = buf;
  p.num_splits = num_splits;
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
  // Chunks per wave unit: enough units to give every CU ~16 waves at the
  // largest batch, but at most 8 chunks so a unit stays a short stream.
  const int64_t tiles = (static_cast<int64_t>(max_tokens) + kExpandTile - 1) / kExpandTile + max_loras;
  int64_t cpr = tiles * total_chunks / (static_cast<int64_t>(num_cus) * 16);
  cpr = cpr < 1 ? 1 : (cpr > 8 ? 8 : cpr);
  p.chunks_per_range = static_cast<int>(cpr);
  int ranges = 0;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) {
    if (s < num_slices) {
      const int chunks = (slice_sizes[s] + kExpandCols - 1) / kExpandCols;
      ranges += (chunks + p.chunks_per_range - 1) / p.chunks_per_range;
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
  p.max_tokens = max_tokens;
  p.max_loras = max_loras;

  const int64_t wave_units = tiles * ranges;
  int64_t grid = (wave_units + kExpandWaves - 1) / kExpandWaves;
  const int64_t cap = static_cast<int64_t>(num_cus) * 16;
  grid = grid < cap ? grid : cap;
  grid = grid < 1 ? 1 : grid;
  switch (rank) {
    case 8: return launch_expand_rank<8>(p, static_cast<int>(grid), stream);
    case 16: return launch_expand_rank<16>(p, static_cast<int>(grid), stream);
    case 32: return launch_expand_rank<32>(p, static_cast<int>(grid), stream);
    default: return launch_expand_rank<64>(p, static_cast<int>(grid), stream);
  }
}

}  // namespace lora
