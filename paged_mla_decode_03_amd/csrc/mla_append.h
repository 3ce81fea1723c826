// Parameters and launch shape of the cache append kernel.
#pragma once

#include <stdint.h>

#include "mla_kernels.h"

namespace mla {

constexpr int kAppendThreads = 256;

struct AppendParams {
  const uint16_t* kv_new;      // [batch][s_new][h_kv][576]
  void* kv;                    // [num_pages][64][h_kv][576] bf16, or fp8 codes
  const int32_t* block_table;  // [batch][max_pages]
  const int32_t* seqlens;      // [batch], tokens cached before the append
  int32_t* bad_rows;           // optional counter of rows without a valid page
  float inv_scale;             // fp8 cache: 1 / its scale (unused for bf16)
  int batch, s_new, h_kv, max_pages, num_pages;
  int chunks;                  // batch * s_new * h_kv * kChunksPerRow
};

__global__ void mla_append_kernel(AppendParams p);
__global__ void mla_append_fp8_kernel(AppendParams p);

}  // namespace mla
