// Parameters of the output projection over all heads (u = W^O [o_1; ...; o_n]).
#pragma once

#include <stdint.h>

namespace mla {

constexpr int kOutProjWaves = 8;       // each over an eighth of the workgroup's K slice
constexpr int kOutProjThreads = kOutProjWaves * 64;
constexpr int kOutProjTileN = 128;     // output columns per workgroup
constexpr int kOutProjTileT = 64;      // tokens per workgroup
constexpr int kNumXcdOutProj = 8;      // MI355X: 8 XCDs, round-robin block dispatch
constexpr int kOutProjMaxSplits = 8;

struct OutProjParams {
  const uint16_t* a;      // bf16 [T][K]: per-head outputs, head-major
  const uint16_t* w;      // bf16 [N][K]: W^O
  uint16_t* out;          // bf16 [T][N]
  float* partial;         // fp32 [splits][T][N] when splits > 1
  int T, K, N;
  int ntiles, tchunks, splits;
};

__global__ void mla_outproj_kernel(OutProjParams p);
__global__ void mla_outproj_reduce_kernel(OutProjParams p);

}  // namespace mla
