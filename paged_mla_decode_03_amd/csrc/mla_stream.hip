// Measurement helpers (gfx950), not steps of the method.
//
// A plain streaming read of device memory, for measurement: the
// rate it reaches is the achievable HBM read bandwidth that the decode's
// rooflines are set beside (the 8 TB/s of the specification is not reached
// by any access pattern).  One 512-thread workgroup per CU reads 64 KB
// contiguous runs, each lane keeping eight 16-byte non-temporal loads in
// flight (64 KB per CU: a probe of this chip reached 7.2 TB/s from 32 KB in
// flight per CU, 4.2 TB/s at 8 KB, and less again with eight such
// workgroups per CU).  The values are folded and stored only if they match
// a pattern no test buffer holds, so the loads stay live.
#include <hip/hip_runtime.h>

#include "mla_kernels.h"

namespace mla {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void mla_stream_read_kernel(const uint4* __restrict__ src_, size_t n16,
                                                                      uint4* sink) {
  constexpr int kDepth = 8;
  constexpr size_t kRun = (size_t)kDepth * kStreamThreads;      // 16-byte elements per run
  const u32x4v* src = (const u32x4v*)src_;
  const size_t runs = n16 / kRun;
  u32x4v acc = {0, 0, 0, 0};
  for (size_t r = blockIdx.x; r < runs; r += gridDim.x) {
    const u32x4v* base = src + r * kRun + threadIdx.x;
    u32x4v v[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) v[k] = __builtin_nontemporal_load(base + k * kStreamThreads);
#pragma unroll
    for (int k = 0; k < kDepth; ++k) acc ^= v[k];
  }
  // The tail after the last whole run.
  for (size_t i = runs * kRun + (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kStreamThreads)
    acc ^= src[i];
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[0] = uint4{acc[0], acc[1], acc[2], acc[3]};
}

// The rate at which one wave reads LDS.  Each wave of a workgroup issues
// 64 * iters reads of one kind, every lane a consecutive 4, 8 or 16 bytes
// (conflict-free), kAhead reads in flight in a ring of registers, and the
// workgroup's first wave records the shader-clock cycles (s_memtime) its
// loop took.  Kinds: 0 ds_read_b128, 1 ds_read_b64, 2 ds_read_b64_tr_b16
// (the transposing read the decode takes V with), 3 ds_read_b32.  The decode
// kernels' K, V and P fragment reads are of kinds 0 and 2; whether a stream
// of them keeps the matrix core fed depends on this rate.
namespace {

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef short s16x4v __attribute__((ext_vector_type(4)));

template <int kKind>
__device__ inline u32x4v lds_read_kind(uint32_t a) {
  if constexpr (kKind == 0) {
    return *(__attribute__((address_space(3))) const u32x4v*)a;
  } else if constexpr (kKind == 1) {
    const u32x2v v = *(__attribute__((address_space(3))) const u32x2v*)a;
    return u32x4v{v[0], v[1], 0u, 0u};
  } else if constexpr (kKind == 2) {
    const s16x4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4v*)a);
    const u32x2v w = __builtin_bit_cast(u32x2v, v);
    return u32x4v{w[0], w[1], 0u, 0u};
  } else {
    const uint32_t v = *(__attribute__((address_space(3))) const uint32_t*)a;
    return u32x4v{v, 0u, 0u, 0u};
  }
}

}  // namespace

template <int kKind, int kWavesIn>
__global__ __launch_bounds__(kWavesIn * 64) void mla_lds_rate_kernel(int iters, long long* cycles, uint4* sink) {
  constexpr int kAhead = 8;
  __shared__ __attribute__((aligned(1024))) char buf[kLdsRateBytes];
  const int tid = threadIdx.x;
  for (int i = tid * 16; i < kLdsRateBytes; i += kWavesIn * 64 * 16)
    *(u32x4v*)(buf + i) = u32x4v{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  // Read r of a wave: the 1 KB run (r + wave) % 64; lane l at byte 16 l of it.
  const uint32_t base = (uint32_t)(uintptr_t)buf + (uint32_t)(lane * 16);
  auto at = [&](int r) __attribute__((always_inline)) { return base + (uint32_t)(((r + wave) & 63) * 1024); };
  u32x4v acc = {0, 0, 0, 0};
  u32x4v ring[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) ring[j] = lds_read_kind<kKind>(at(j));
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      acc ^= ring[j % kAhead];
      ring[j % kAhead] = lds_read_kind<kKind>(at(j + kAhead + it));
    }
  }
#pragma unroll
  for (int j = 0; j < kAhead; ++j) acc ^= ring[j];
  const long long t1 = __builtin_amdgcn_s_memtime();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[0] = uint4{acc[0], acc[1], acc[2], acc[3]};
}

template __global__ void mla_lds_rate_kernel<0, 4>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<1, 4>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<2, 4>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<3, 4>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<0, 8>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<1, 8>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<2, 8>(int, long long*, uint4*);
template __global__ void mla_lds_rate_kernel<3, 8>(int, long long*, uint4*);

}  // namespace mla
