// Parameters of the per-head projections around the decode kernel.
#pragma once

#include <stdint.h>

namespace mla {

constexpr int kAbsorbThreads = 256;   // 4 waves, 16 output columns each
constexpr int kAbsorbTileN = 64;
constexpr int kAbsorbTileT = 64;
constexpr int kDh = 128;              // per-head q^C / k^C / v^C width
constexpr int kDr = 64;               // RoPE part of a query head

// C[t][h][n] = sum_k A[t][h][k] * Bt[h][n][k], bf16 in, fp32 accumulate, bf16 out.
struct AbsorbParams {
  const uint16_t* a;      // element (t, h, k) at a[t * a_t + h * K + k]
  const uint16_t* bt;     // element (h, n, k) at bt[(h * N + n) * K + k]
  uint16_t* c;            // element (t, h, n) at c[t * c_t + h * c_h + n]
  const uint16_t* rope;   // optional [T][H][64], copied to c[t][h][N .. N + 64)
  int T, H;
  long long a_t, c_t;
  int c_h;
};

template <int K, int N>
__global__ void mla_absorb_kernel(AbsorbParams p);

}  // namespace mla
