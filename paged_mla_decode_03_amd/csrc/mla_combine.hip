// Log-sum-exp merge of split-KV partials (gfx950).
//
// The deepseek.csdn.net FlashMLA article (section 4.2(1)) pairs the split-KV
// forward kernel with a kernel that merges the per-split results.  Each split
// s of a query row left O_s (normalised by its own softmax sum) and lse_s;
// the merge is exact:
//     lse = M + ln sum_s exp(lse_s - M),  M = max_s lse_s
//     O   = sum_s exp(lse_s - lse) * O_s
// Splits whose keys were all masked carry lse_s = -inf and weigh nothing; a
// row with no visible key at all gets O = 0, lse = -inf.
//
// Two variants, chosen on the host from the number of workers per sequence:
//   * mla_combine_kernel, one wave per (sequence, latent head, query row),
//     four rows per workgroup, for launches where sequences split a few ways
//     (workers <= 2 x sequences): each lane owns 8 of the 512 columns, and
//     the first four splits' rows are loaded together before any reduction;
//   * mla_combine_wide_kernel, one workgroup of four waves per row, for
//     launches with few sequences over many workers (one long sequence
//     spread over most of the chip splits ~100 ways), so that a row has four
//     waves' loads in flight instead of one:
//   1. every thread takes splits tid, tid + 256, ... for the maximum M and
//      then for sum_s exp(lse_s - M) (workgroup reductions through LDS);
//   2. wave w sums the partial rows of splits w, w + 4, w + 8, ..., each lane
//      owning 8 of the 512 columns, with up to kInFlight splits' loads issued
//      before their multiply-adds;
//   3. the four waves' sums are added in wave order through LDS.
// In both, every split goes to a fixed wave and every sum has a fixed order,
// so the result does not depend on scheduling.  Sequences with a single split were
// finished by the decode kernel and are skipped.
#include "mla_kernels.h"

namespace mla {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineWaves = kCombineThreads / 64;
constexpr int kInFlight = 4;   // splits per wave whose partial rows are loaded together

__device__ inline float wave_reduce_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ inline float wave_reduce_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

}  // namespace

__global__ __launch_bounds__(kCombineThreads) void mla_combine_wide_kernel(CombineParams p) {
  __shared__ float red[kCombineWaves];
  __shared__ __attribute__((aligned(16))) f32x4 part[kCombineWaves - 1][64][2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int task = blockIdx.x;
  const int per_seq = p.h_kv * p.rows;
  const int b = task / per_seq;
  const int g = (task - b * per_seq) / p.rows;
  const int row = task - b * per_seq - g * p.rows;
  const int s0 = p.num_splits[b];
  const int n = p.num_splits[b + 1] - s0;
  if (n == 1) return;

  const int tok = row / p.group;
  const int head = g * p.group + (row - tok * p.group);
  uint16_t* op = p.o + ((size_t)(b * p.s_q + tok) * p.h_q + head) * kDv + lane * 8;
  float* lp = p.lse + ((size_t)b * p.h_q + head) * p.s_q + tok;
  // lse_s of split s sits at lse0[s * stride]; its O_s row at o0 + s * stride * kDv.
  const size_t stride = (size_t)p.h_kv * p.rows;
  const float* lse0 = p.ws_lse + (size_t)(s0 * p.h_kv + g) * p.rows + row;
  const float* o0 = p.ws_o + ((size_t)(s0 * p.h_kv + g) * p.rows + row) * kDv + lane * 8;

  // 1. M = max_s lse_s, then Z = sum_s exp(lse_s - M).
  float m = -__builtin_huge_valf();
  for (int i = tid; i < n; i += kCombineThreads) m = fmaxf(m, lse0[(size_t)i * stride]);
  m = wave_reduce_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kCombineWaves; ++w) M = fmaxf(M, red[w]);
  if (n == 0 || M == -__builtin_huge_valf()) {
    if (wave == 0) {
      *(uint4*)op = uint4{0, 0, 0, 0};
      if (lane == 0) *lp = -__builtin_huge_valf();
    }
    return;
  }
  __syncthreads();   // every wave has read red[] before it is reused
  float z = 0.f;
  for (int i = tid; i < n; i += kCombineThreads) z += expf(lse0[(size_t)i * stride] - M);
  z = wave_reduce_sum(z);
  if (lane == 0) red[wave] = z;
  __syncthreads();
  float Z = red[0];
#pragma unroll
  for (int w = 1; w < kCombineWaves; ++w) Z += red[w];
  const float lse = M + logf(Z);

  // 2. This wave's splits: wave, wave + W, wave + 2W, ... (W = 4 waves).
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int base = wave; base < n; base += kCombineWaves * kInFlight) {
    f32x4 v[kInFlight][2];
    float wgt[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int sidx = base + k * kCombineWaves;
      if (sidx < n) {
        const f32x4* src = (const f32x4*)(o0 + (size_t)sidx * stride * kDv);
        v[k][0] = src[0];
        v[k][1] = src[1];
        wgt[k] = lse0[(size_t)sidx * stride];
      } else {
        v[k][0] = v[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        wgt[k] = -__builtin_huge_valf();
      }
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const float w = expf(wgt[k] - lse);   // exp(-inf) = 0 past n
      a0 += w * v[k][0];
      a1 += w * v[k][1];
    }
  }

  // 3. Sum the waves' rows in wave order.
  if (wave > 0) {
    part[wave - 1][lane][0] = a0;
    part[wave - 1][lane][1] = a1;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kCombineWaves - 1; ++w) {
      a0 += part[w][lane][0];
      a1 += part[w][lane][1];
    }
    uint4 out;
    out.x = pack_bf16x2(a0[0], a0[1]);
    out.y = pack_bf16x2(a0[2], a0[3]);
    out.z = pack_bf16x2(a1[0], a1[1]);
    out.w = pack_bf16x2(a1[2], a1[3]);
    *(uint4*)op = out;
    if (lane == 0) *lp = lse;
  }
}


__global__ __launch_bounds__(kCombineRowsPerWaveBlock * 64) void mla_combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * kCombineRowsPerWaveBlock + (threadIdx.x >> 6);
  const int per_seq = p.h_kv * p.rows;
  if (task >= p.batch * per_seq) return;
  const int b = task / per_seq;
  const int g = (task - b * per_seq) / p.rows;
  const int row = task - b * per_seq - g * p.rows;
  const int s0 = p.num_splits[b];
  const int n = p.num_splits[b + 1] - s0;
  if (n == 1) return;

  const int tok = row / p.group;
  const int head = g * p.group + (row - tok * p.group);
  uint16_t* op = p.o + ((size_t)(b * p.s_q + tok) * p.h_q + head) * kDv + lane * 8;
  float* lp = p.lse + ((size_t)b * p.h_q + head) * p.s_q + tok;
  // lse_s of split s sits at lse0[s * stride]; its O_s row at o0 + s * stride * kDv.
  const size_t stride = (size_t)p.h_kv * p.rows;
  const float* lse0 = p.ws_lse + (size_t)(s0 * p.h_kv + g) * p.rows + row;
  const float* o0 = p.ws_o + ((size_t)(s0 * p.h_kv + g) * p.rows + row) * kDv + lane * 8;

  // The first four splits' lse values and partial rows are loaded together,
  // before any reduction, so a row with up to four splits costs one memory
  // round trip; splits past the fourth follow four (then two) at a time.
  constexpr int kFirst = 4;
  f32x4 v0[kFirst][2];
  float l0[kFirst];
#pragma unroll
  for (int k = 0; k < kFirst; ++k) {
    if (k < n) {
      const f32x4* src = (const f32x4*)(o0 + (size_t)k * stride * kDv);
      v0[k][0] = *(src);
      v0[k][1] = *(src + 1);
      l0[k] = lse0[(size_t)k * stride];
    } else {
      v0[k][0] = v0[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      l0[k] = -__builtin_huge_valf();
    }
  }
  float M = fmaxf(fmaxf(l0[0], l0[1]), fmaxf(l0[2], l0[3]));   // the same in every lane
  if (n > kFirst) {
    float m = -__builtin_huge_valf();
    for (int i = kFirst + lane; i < n; i += 64) m = fmaxf(m, lse0[(size_t)i * stride]);
    M = fmaxf(M, wave_reduce_max(m));
  }
  if (n == 0 || M == -__builtin_huge_valf()) {
    *(uint4*)op = uint4{0, 0, 0, 0};
    if (lane == 0) *lp = -__builtin_huge_valf();
    return;
  }
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kFirst; ++k) z += expf(l0[k] - M);   // exp(-inf) = 0 past n
  if (n > kFirst) {
    float zr = 0.f;
    for (int i = kFirst + lane; i < n; i += 64) zr += expf(lse0[(size_t)i * stride] - M);
    z += wave_reduce_sum(zr);
  }
  const float lse = M + logf(z);

  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kFirst; ++k) {
    const float w = expf(l0[k] - lse);
    a0 += w * v0[k][0];
    a1 += w * v0[k][1];
  }
  int i = kFirst;
  for (; i + 4 <= n; i += 4) {
    f32x4 v[4][2];
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4* src = (const f32x4*)(o0 + (size_t)(i + k) * stride * kDv);
      v[k][0] = *(src);
      v[k][1] = *(src + 1);
      w[k] = expf(lse0[(size_t)(i + k) * stride] - lse);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a0 += w[k] * v[k][0];
      a1 += w[k] * v[k][1];
    }
  }
  if (i + 2 <= n) {
    f32x4 v[2][2];
    float w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const f32x4* src = (const f32x4*)(o0 + (size_t)(i + k) * stride * kDv);
      v[k][0] = *(src);
      v[k][1] = *(src + 1);
      w[k] = expf(lse0[(size_t)(i + k) * stride] - lse);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      a0 += w[k] * v[k][0];
      a1 += w[k] * v[k][1];
    }
    i += 2;
  }
  if (i < n) {
    const f32x4* src = (const f32x4*)(o0 + (size_t)i * stride * kDv);
    const float w = expf(lse0[(size_t)i * stride] - lse);
    a0 += w * *(src);
    a1 += w * *(src + 1);
  }
  uint4 v;
  v.x = pack_bf16x2(a0[0], a0[1]);
  v.y = pack_bf16x2(a0[2], a0[3]);
  v.z = pack_bf16x2(a1[0], a1[1]);
  v.w = pack_bf16x2(a1[2], a1[3]);
  *(uint4*)op = v;
  if (lane == 0) *lp = lse;
}

}  // namespace mla
