// CPU oracle for the multi-LoRA shrink/expand path.
//
// TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
// benchmark's CPU-baseline leg load this library; the GPU path never does, and
// the two share no source, header, helper or table.
//
// What is computed, written as the plain definitions with fp64 accumulation and
// per-token loops:
//
//  * metadata: the token -> adapter map of an ungrouped batch is turned into a
//    stable grouping of token indices by adapter id, with per-adapter counts
//    and start offsets.  vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1"
//    (section "Why do we need a new set of kernels") describes the ungrouped V1
//    batch whose kernels must know which tokens map to which LoRA id; the
//    MLC-LLM issue "[Tracking] Multi-LoRA Serving" (Overview) describes
//    Punica's segment vector, i.e. which rows of one batch belong to which
//    request.  Reading: ids outside [-1, max_loras) count as -1 (no adapter);
//    groups are ordered by ascending id with the no-adapter group first; the
//    active list holds the ids >= 0 that occur, ascending, and unused slots
//    hold (-1, 0, num_tokens).
//  * shrink: buf[s][t][k] = scale * sum_h x[t][h] * A_s[l][k][h] for every
//    token t with adapter l >= 0 (the "shrink" half of the low-rank product
//    named in PR #13096's summary; the low-rank multiplication per segment in
//    the MLC-LLM issue's Overview).
//  * expand: y[t][off_s + n] = y0[t][off_s + n] + sum_k buf[s][t][k] *
//    B_s[l][n][k], with off_s the running sum of the slice widths (the
//    "expand" half).  Tokens without an adapter keep y0.  The bf16 result is
//    the fp64 value rounded once to the nearest bfloat16, ties to even.
//
// Layouts: x [num_tokens][ldx]; A_s [max_loras][rank][hidden];
// B_s [max_loras][n_s][rank]; y [num_tokens][ldy]; bf16 values are raw uint16
// bit patterns.  Returns 0 on success, 1 on an invalid argument.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

double widen_bf16(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// The bfloat16 value nearest to v (ties to the even significand), taken
// straight from the double: 8 significant bits in float32's exponent range,
// quantum 2^-133 below the smallest normal 2^-126, overflow to infinity.
uint16_t nearest_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return sign | 0x7F80;
  int e = 0;
  std::frexp(a, &e);                      // a = m * 2^e, m in [0.5, 1)
  const int q = std::max(e - 8, -133);    // exponent of one unit in the last place
  const double r = std::nearbyint(std::ldexp(a, -q));  // default mode: nearest, ties even
  const double res = std::ldexp(r, q);
  if (res >= 0x1p128) return sign | 0x7F80;
  const float f = static_cast<float>(res);  // exact: at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return sign | static_cast<uint16_t>(u >> 16);
}

int adapter_of(const int32_t* mapping, int64_t t, int32_t max_loras) {
  const int32_t m = mapping[t];
  return (m >= -1 && m < max_loras) ? m : -1;
}

template <class F>
void for_token_ranges(int64_t num_tokens, int32_t num_threads, F&& body) {
  int64_t n = num_threads > 0 ? num_threads
                              : static_cast<int64_t>(std::thread::hardware_concurrency());
  n = std::max<int64_t>(1, std::min<int64_t>(n, num_tokens));
  if (n == 1) {
    body(int64_t{0}, num_tokens);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) {
    const int64_t lo = num_tokens * i / n, hi = num_tokens * (i + 1) / n;
    pool.emplace_back([&body, lo, hi] { body(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

uint16_t oracle_round_bf16(double v) { return nearest_bf16(v); }

double oracle_widen_bf16(uint16_t bits) { return widen_bf16(bits); }

int oracle_default_threads(void) {
  return static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
}

// sorted_token_ids: [num_tokens]; the four per-slot arrays: [max_loras].
int oracle_prepare_metadata(const int32_t* mapping, int32_t num_tokens, int32_t max_loras,
                            int32_t* sorted_token_ids, int32_t* active_lora_ids,
                            int32_t* num_tokens_per_lora, int32_t* lora_token_start,
                            int32_t* num_active) {
  if (num_tokens < 0 || max_loras < 1) return 1;
  if (num_tokens > 0 && (!mapping || !sorted_token_ids)) return 1;
  if (!active_lora_ids || !num_tokens_per_lora || !lora_token_start || !num_active) return 1;

  // Group g = id + 1, so the no-adapter group (id -1) is group 0.
  std::vector<int64_t> count(static_cast<size_t>(max_loras) + 1, 0);
  for (int64_t t = 0; t < num_tokens; ++t) ++count[adapter_of(mapping, t, max_loras) + 1];

  std::vector<int64_t> start(count.size(), 0);
  int64_t running = 0;
  for (size_t g = 0; g < count.size(); ++g) {
    start[g] = running;
    running += count[g];
  }

  // Visiting tokens in index order keeps equal ids in index order (stability).
  std::vector<int64_t> cursor = start;
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int g = adapter_of(mapping, t, max_loras) + 1;
    sorted_token_ids[cursor[g]++] = static_cast<int32_t>(t);
  }

  int32_t na = 0;
  for (int32_t l = 0; l < max_loras; ++l) {
    if (count[l + 1] == 0) continue;
    active_lora_ids[na] = l;
    num_tokens_per_lora[na] = static_cast<int32_t>(count[l + 1]);
    lora_token_start[na] = static_cast<int32_t>(start[l + 1]);
    ++na;
  }
  for (int32_t i = na; i < max_loras; ++i) {
    active_lora_ids[i] = -1;
    num_tokens_per_lora[i] = 0;
    lora_token_start[i] = num_tokens;
  }
  *num_active = na;
  return 0;
}

// buf: [num_slices][num_tokens][rank]; rows of tokens without an adapter are
// not written.
int oracle_shrink(const uint16_t* x, int64_t ldx, int32_t num_tokens, int32_t hidden,
                  const uint16_t* const* lora_a, int32_t num_slices, int32_t rank, double scale,
                  const int32_t* mapping, int32_t max_loras, double* buf, int32_t num_threads) {
  if (num_tokens < 0 || hidden < 1 || num_slices < 1 || rank < 1 || max_loras < 1) return 1;
  if (ldx < hidden) return 1;
  if (num_tokens == 0) return 0;
  if (!x || !lora_a || !mapping || !buf) return 1;
  for (int32_t s = 0; s < num_slices; ++s)
    if (!lora_a[s]) return 1;

  for_token_ranges(num_tokens, num_threads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      const int l = adapter_of(mapping, t, max_loras);
      if (l < 0) continue;
      const uint16_t* xrow = x + t * ldx;
      for (int32_t s = 0; s < num_slices; ++s) {
        for (int32_t k = 0; k < rank; ++k) {
          const uint16_t* arow = lora_a[s] + (static_cast<int64_t>(l) * rank + k) * hidden;
          double acc = 0.0;
          for (int32_t h = 0; h < hidden; ++h) acc += widen_bf16(xrow[h]) * widen_bf16(arow[h]);
          buf[(static_cast<int64_t>(s) * num_tokens + t) * rank + k] = scale * acc;
        }
      }
    }
  });
  return 0;
}

// y64 and y_bf16: [num_tokens][ldy].  Columns past the last slice, and whole
// rows of tokens without an adapter, are copies of y0.
int oracle_expand(const double* buf, const uint16_t* const* lora_b, const int32_t* slice_sizes,
                  int32_t num_slices, int32_t rank, const uint16_t* y0, int64_t ldy,
                  const int32_t* mapping, int32_t num_tokens, int32_t max_loras, double* y64,
                  uint16_t* y_bf16, int32_t num_threads) {
  if (num_tokens < 0 || num_slices < 1 || rank < 1 || max_loras < 1 || !slice_sizes) return 1;
  int64_t n_total = 0;
  for (int32_t s = 0; s < num_slices; ++s) {
    if (slice_sizes[s] < 0) return 1;
    n_total += slice_sizes[s];
  }
  if (ldy < n_total) return 1;
  if (num_tokens == 0) return 0;
  if (!buf || !lora_b || !y0 || !mapping || !y64 || !y_bf16) return 1;
  for (int32_t s = 0; s < num_slices; ++s)
    if (!lora_b[s]) return 1;

  for_token_ranges(num_tokens, num_threads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      const uint16_t* yin = y0 + t * ldy;
      double* yout = y64 + t * ldy;
      uint16_t* ybits = y_bf16 + t * ldy;
      for (int64_t c = 0; c < ldy; ++c) {
        yout[c] = widen_bf16(yin[c]);
        ybits[c] = yin[c];
      }
      const int l = adapter_of(mapping, t, max_loras);
      if (l < 0) continue;
      int64_t off = 0;
      for (int32_t s = 0; s < num_slices; ++s) {
        const int32_t n_s = slice_sizes[s];
        const double* brow = buf + (static_cast<int64_t>(s) * num_tokens + t) * rank;
        for (int32_t n = 0; n < n_s; ++n) {
          const uint16_t* wrow = lora_b[s] + (static_cast<int64_t>(l) * n_s + n) * rank;
          double delta = 0.0;
          for (int32_t k = 0; k < rank; ++k) delta += brow[k] * widen_bf16(wrow[k]);
          const double v = widen_bf16(yin[off + n]) + delta;
          yout[off + n] = v;
          ybits[off + n] = nearest_bf16(v);
        }
        off += n_s;
      }
    }
  });
  return 0;
}

}  // extern "C"
