// Shrink step: buf_p[s][t][k] = scale * sum_{h in part p} x[t][h] * A_s[l][k][h]
// for every token t with adapter l, read through the grouped token order.
//
// vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1": the summary names the
// shrink kernel; "Kernel Code Change" item 2 is the gather of the input tokens
// through the token -> LoRA map.  MLC-LLM issue "[Tracking] Multi-LoRA
// Serving", Overview: one launch covers every segment, each with its own
// low-rank weights.
//
// gfx950 mapping.  A work unit is (tile of 16 grouped tokens of one adapter,
// part p of the hidden dimension).  Each unit is a dense 16-token x (S*r)-output
// contraction, computed on the matrix cores as D^T = A . x^T with
// v_mfma_f32_16x16x32_bf16: the M dimension is the S*r outputs (blocks of 16),
// N the 16 tokens, K the hidden dimension.  The sum over K is order-free, so
// lane group g (lanes 16g..16g+15) feeds MFMA i of a 64-wide chunk with the
// elements [16g + 8i, 16g + 8i + 8) of that chunk for BOTH operands: every lane
// then reads 32 contiguous bytes of its token's x row and of its A row, the
// four lane groups together one 128-byte line per row.  The four waves of a
// workgroup take interleaved chunks of the part and are summed through LDS in a
// fixed order, so results are bit-identical run to run.  The grid is fixed by
// the size arguments; workgroups stride over the units of the actual batch.

#include "device_common.hpp"

namespace lora {

constexpr int kShrinkThreads = 256;
constexpr int kShrinkWaves = kShrinkThreads / kWave;
constexpr int kShrinkTile = 16;   // tokens per unit (the MFMA N dimension)
constexpr int kShrinkChunk = 64;  // hidden elements per wave step (two MFMA K-steps)

struct ShrinkParams {
  const uint16_t* x;
  int64_t ldx;
  int hidden;
  const uint16_t* a[LORA_MAX_SLICES];
  int num_slices;
  int rank;
  float scale;
  float* buf;
  int num_splits;
  int split_len;  // hidden elements per part, a multiple of kShrinkChunk
  const int32_t* sorted;
  const int32_t* active_ids;
  const int32_t* counts;
  const int32_t* starts;
  const int32_t* num_active;
  int max_tokens;
  int max_loras;
};

__device__ __forceinline__ const uint16_t* slice_ptr(const ShrinkParams& p, int s) {
  // select chain: per-lane slice index must not index the kernel-argument array
  const uint16_t* r = p.a[0];
  r = s == 1 ? p.a[1] : r;
  r = s == 2 ? p.a[2] : r;
  r = s == 3 ? p.a[3] : r;
  return r;
}

// NB = number of 16-output blocks covering num_slices * rank outputs.
template <int NB>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkParams p) {
  __shared__ SegmentTable tab;
  __shared__ f32x4 partial[kShrinkWaves - 1][NB][kWave];

  build_segment_table<kShrinkTile>(tab, p.active_ids, p.counts, p.starts, p.num_active,
                                   p.max_loras, p.max_tokens);
  const int num_tiles = tab.num_tiles;
  const int units = num_tiles * p.num_splits;

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;  // token within the tile (MFMA N index)
  const int grp = lane >> 4;  // lane group: K sub-range, and output rows 4*grp..4*grp+3
  const int nout = p.num_slices * p.rank;

  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int part = u / num_tiles;
    const int m = u - part * num_tiles;
    const Tile tile = resolve_tile<kShrinkTile>(tab, m);

    const int t = col < tile.rows ? token_at(p.sorted, tile.first + col, p.max_tokens) : -1;
    const uint16_t* xrow = t >= 0 ? p.x + static_cast<int64_t>(t) * p.ldx : nullptr;

    // A-operand rows: output o = 16*nb + col of this lane's MFMA M index.
    const uint16_t* arow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int o = 16 * nb + col;
      arow[nb] = nullptr;
      if (o < nout) {
        const int s = o / p.rank;
        const int k = o - s * p.rank;
        arow[nb] = slice_ptr(p, s) + (static_cast<int64_t>(tile.lora) * p.rank + k) * p.hidden;
      }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int kbeg = part * p.split_len;
    const int kend = min(p.hidden, kbeg + p.split_len);
    for (int kc = kbeg + wave * kShrinkChunk; kc < kend; kc += kShrinkWaves * kShrinkChunk) {
      u32x4 xv[2];
      u32x4 av[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = kc + 16 * grp + 8 * i;
        const bool in = k < kend;  // kend is a multiple of 8: a piece is wholly in or out
        xv[i] = (in && xrow) ? load16(xrow + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          av[nb][i] = (in && arow[nb]) ? load16(arow[nb] + k) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av[nb][i]), __builtin_bit_cast(bf16x8, xv[i]),
              acc[nb], 0, 0, 0);
      }
    }

    if (wave > 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) partial[wave - 1][nb][lane] = acc[nb];
    }
    __syncthreads();
    if (wave == 0 && t >= 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 v = acc[nb];
#pragma unroll
        for (int w = 0; w < kShrinkWaves - 1; ++w) v += partial[w][nb][lane];
        // D^T layout: this lane holds outputs o = 16*nb + 4*grp + j (j = 0..3)
        // of token column `col`; rank is a multiple of 8, so the four share a slice.
        const int o = 16 * nb + 4 * grp;
        if (o < nout) {
          const int s = o / p.rank;
          const int k = o - s * p.rank;
          v *= p.scale;
          float* dst = p.buf + ((static_cast<int64_t>(part) * p.num_slices + s) * p.max_tokens + t) *
                                   p.rank + k;
          store16(dst, __builtin_bit_cast(u32x4, v));
        }
      }
    }
    __syncthreads();
  }
}

template <int NB>
hipError_t launch_shrink_nb(const ShrinkParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(shrink_kernel<NB>, dim3(grid), dim3(kShrinkThreads), 0, stream, p);
  return hipGetLastError();
}

int shrink_split_len(int hidden, int num_splits) {
  const int per = (hidden + num_splits - 1) / num_splits;
  return (per + kShrinkChunk - 1) / kShrinkChunk * kShrinkChunk;
}

int shrink_grid(int max_tokens, int max_loras, int num_splits, int num_cus) {
  const int64_t tiles = (static_cast<int64_t>(max_tokens) + kShrinkTile - 1) / kShrinkTile + max_loras;
  const int64_t units = tiles * num_splits;
  const int64_t cap = static_cast<int64_t>(num_cus) * 8;
  return static_cast<int>(units < cap ? units : cap);
}

hipError_t launch_shrink(const uint16_t* x, int64_t ldx, int hidden, const uint16_t* const* lora_a,
                         int num_slices, int rank, float scale, float* buf, int num_splits,
                         const lora_meta_t& meta, int max_tokens, int max_loras, int num_cus,
                         hipStream_t stream) {
  ShrinkParams p{};
  p.x = x;
  p.ldx = ldx;
  p.hidden = hidden;
  for (int s = 0; s < LORA_MAX_SLICES; ++s) p.a[s] = s < num_slices ? lora_a[s] : lora_a[0];
  p.num_slices = num_slices;
  p.rank = rank;
  p.scale = scale;
  p.buf = buf;
  p.num_splits = num_splits;
  p.split_len = shrink_split_len(hidden, num_splits);
  p.sorted = meta.sorted_token_ids;
  p.active_ids = meta.active_lora_ids;
  p.counts = meta.num_tokens_per_lora;
  p.starts = meta.lora_token_start;
  p.num_active = meta.num_active;
  p.max_tokens = max_tokens;
  p.max_loras = max_loras;
  const int grid = shrink_grid(max_tokens, max_loras, num_splits, num_cus);
  const int nb = (num_slices * rank + 15) / 16;
  switch (nb) {
    case 1: return launch_shrink_nb<1>(p, grid, stream);
    case 2: return launch_shrink_nb<2>(p, grid, stream);
    case 3: return launch_shrink_nb<3>(p, grid, stream);
    case 4: return launch_shrink_nb<4>(p, grid, stream);
    case 5:
    case 6: return launch_shrink_nb<6>(p, grid, stream);
    case 7:
    case 8: return launch_shrink_nb<8>(p, grid, stream);
    case 9:
    case 10:
    case 11:
    case 12: return launch_shrink_nb<12>(p, grid, stream);
    default: return launch_shrink_nb<16>(p, grid, stream);
  }
}

}  // namespace lora
