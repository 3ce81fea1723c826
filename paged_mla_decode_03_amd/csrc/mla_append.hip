// Append of new tokens' latent rows to the paged cache.
//
// The cache keeps the [c^KV; k^R] row of every token already seen, so a
// decode step computes only the new token's row and adds it (deepseek.csdn.net
// FlashMLA article, section 4.1); the cache is a pool of 64-slot pages mapped
// through block_table (same article, section 4.2(1)).  New token i of
// sequence b takes logical position L_b + i, L_b = cache_seqlens[b]: page
// block_table[b][(L_b + i) / 64], slot (L_b + i) % 64.
//
// A copy, bound by HBM and, at decode sizes, by the launch itself: one
// thread moves one 16-byte chunk of a row (72 per row), so each wave reads
// and writes 1 KB of consecutive bytes and no byte is touched twice.  A row
// whose position has no valid page (negative length, past the block table,
// page id outside the pool) is not written; it is counted in bad_rows.
//
// mla_append_fp8_kernel writes the same rows into an fp8 cache (OCP E4M3,
// one fp32 scale per cache): each value x becomes the nearest E4M3 code (ties
// to even) of float(x) * inv_scale clamped to [-448, 448], so a finite input
// never becomes the NaN code (v_cvt_pk_fp8_f32 itself does not saturate); a
// NaN input stays NaN.  One thread reads 16 bytes (8 bf16) and writes 8.
#include <hip/hip_runtime.h>

#include "mla_append.h"

namespace mla {

__global__ __launch_bounds__(kAppendThreads) void mla_append_kernel(AppendParams p) {
  const int t = blockIdx.x * kAppendThreads + threadIdx.x;
  if (t >= p.chunks) return;
  const int row = t / kChunksPerRow;                 // (b * s_new + i) * h_kv + g
  const int chunk = t - row * kChunksPerRow;
  const int g = row % p.h_kv;
  const int bi = row / p.h_kv;
  const int i = bi % p.s_new;
  const int b = bi / p.s_new;
  const int len = p.seqlens[b];
  const long long pos = (long long)len + i;
  const long long blk = pos / kPage;
  int pid = -1;
  if (len >= 0 && blk < p.max_pages) pid = p.block_table[(size_t)b * p.max_pages + blk];
  if (pid < 0 || pid >= p.num_pages) {
    if (chunk == 0 && p.bad_rows) atomicAdd(p.bad_rows, 1);
    return;
  }
  const size_t slot = ((size_t)pid * kPage + (size_t)(pos - blk * kPage)) * p.h_kv + g;
  const uint4 v = reinterpret_cast<const uint4*>(p.kv_new)[(size_t)row * kChunksPerRow + chunk];
  reinterpret_cast<uint4*>(p.kv)[slot * kChunksPerRow + chunk] = v;
}

namespace {

__device__ inline float clamp_e4m3(float v) {
  // |v| <= 448, or NaN passed through (the comparison is false for NaN).
  return fabsf(v) <= 448.0f || v != v ? v : __builtin_copysignf(448.0f, v);
}

}  // namespace

__global__ __launch_bounds__(kAppendThreads) void mla_append_fp8_kernel(AppendParams p) {
  const int t = blockIdx.x * kAppendThreads + threadIdx.x;
  if (t >= p.chunks) return;
  const int row = t / kChunksPerRow;                 // (b * s_new + i) * h_kv + g
  const int chunk = t - row * kChunksPerRow;
  const int g = row % p.h_kv;
  const int bi = row / p.h_kv;
  const int i = bi % p.s_new;
  const int b = bi / p.s_new;
  const int len = p.seqlens[b];
  const long long pos = (long long)len + i;
  const long long blk = pos / kPage;
  int pid = -1;
  if (len >= 0 && blk < p.max_pages) pid = p.block_table[(size_t)b * p.max_pages + blk];
  if (pid < 0 || pid >= p.num_pages) {
    if (chunk == 0 && p.bad_rows) atomicAdd(p.bad_rows, 1);
    return;
  }
  const size_t slot = ((size_t)pid * kPage + (size_t)(pos - blk * kPage)) * p.h_kv + g;
  const uint4 v = reinterpret_cast<const uint4*>(p.kv_new)[(size_t)row * kChunksPerRow + chunk];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t a = w[2 * k], c = w[2 * k + 1];
    const float f0 = clamp_e4m3(__builtin_bit_cast(float, a << 16) * p.inv_scale);
    const float f1 = clamp_e4m3(__builtin_bit_cast(float, a & 0xFFFF0000u) * p.inv_scale);
    const float f2 = clamp_e4m3(__builtin_bit_cast(float, c << 16) * p.inv_scale);
    const float f3 = clamp_e4m3(__builtin_bit_cast(float, c & 0xFFFF0000u) * p.inv_scale);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, r, true);
    out[k] = (uint32_t)r;
  }
  reinterpret_cast<uint2*>(p.kv)[slot * kChunksPerRow + chunk] = uint2{out[0], out[1]};
}

}  // namespace mla
