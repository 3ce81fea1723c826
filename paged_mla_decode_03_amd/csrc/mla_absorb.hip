// Per-head projections around the decode kernel (gfx950).
//
// The decode kernel works in the latent space of the cache (deepseek.csdn.net
// FlashMLA article, section 2.2, the matrix-absorption paragraph): a head's
// query enters as [W^UK^T q^C (512); q^R (64)], since q^C . (W^UK c) =
// (W^UK^T q^C) . c, and its output leaves as the latent sum o = sum_j p_j c_j,
// which W^UV maps to the head's value space, since W^UV is linear and the
// weights p_j are shared.  Both are per-head products with a weight shared by
// all tokens:
//     query:  q~[t][h][0:512] = sum_d q^C[t][h][d] * W^UK[h][d][:]   (K = 128, N = 512)
//     output: u[t][h][0:128]  = sum_c o[t][h][c]  * W^UV[h][:][c]   (K = 512, N = 128)
// with the query weight passed c-major, W^UK^T [h][512][128], so that both
// read their weight rows along K.
//
// At decode sizes (tens to hundreds of tokens) the weights dominate the bytes
// (16.8 MB each for 128 heads) and the products are bound by HBM, not by the
// matrix cores.  A workgroup takes one head, 64 output columns and 64 tokens:
// it stages the 64 token rows in LDS once (and, for the query projection,
// the 64 weight rows too), and wave w computes the 16 x 64 tile of columns
// 16w..16w+15 as D^T = Bt A^T with
// v_mfma_f32_16x16x32_bf16 (weight rows as the A operand, token rows as the
// B operand, both 16-byte reads along K), so each lane ends with 4
// consecutive output columns of one token, stored as 8 bytes.
#include <hip/hip_runtime.h>

#include "mla_absorb.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ inline bf16x8 load8(const uint16_t* p) { return __builtin_bit_cast(bf16x8, *(const uint4*)p); }

}  // namespace

template <int K, int N>
__global__ __launch_bounds__(kAbsorbThreads) void mla_absorb_kernel(AbsorbParams p) {
  static_assert(K % 32 == 0 && N % kAbsorbTileN == 0, "whole tiles");
  // The workgroup's 64 token rows are staged once in LDS (rows padded by 16
  // bytes so that the 16 rows one fragment read touches fall in different
  // banks) and read there by all four waves.  Each wave's 16 weight rows are
  // its own: with K = 512 they go straight from memory into registers (64
  // VGPRs); with K = 128 they are staged in LDS with the token rows, which
  // measured faster at decode sizes (64 tokens: 7.4 against 8.0 us).
  constexpr bool kStageW = K <= 128;
  constexpr int kStride = K + 8;
  constexpr int kW = K / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sa[kAbsorbTileT * kStride];
  __shared__ __attribute__((aligned(16))) uint16_t sw[kStageW ? kAbsorbTileN * kStride : 8];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = blockIdx.y * kAbsorbTileN;
  const int t0 = blockIdx.z * kAbsorbTileT;
  const int col = lane & 15;         // weight row (A operand) / token (B operand) within a tile
  const int kq = 8 * (lane >> 4);    // this lane's 8 values of each 32-wide k step
  bf16x8 wf[kW];
  if constexpr (!kStageW) {
    const uint16_t* wrow = p.bt + ((size_t)h * N + nb + 16 * wave + col) * K + kq;
#pragma unroll
    for (int k = 0; k < kW; ++k) wf[k] = load8(wrow + 32 * k);
  }
  constexpr int kChunks = K / 8;                       // 16-byte chunks per row
  for (int i = threadIdx.x; i < kAbsorbTileT * kChunks; i += kAbsorbThreads) {
    const int r = i / kChunks, c = 8 * (i % kChunks);
    const int t = min(t0 + r, p.T - 1);                  // rows past T repeat row T-1; never stored
    *(uint4*)(sa + r * kStride + c) = *(const uint4*)(p.a + (size_t)t * p.a_t + (size_t)h * K + c);
    if constexpr (kStageW)
      *(uint4*)(sw + r * kStride + c) = *(const uint4*)(p.bt + ((size_t)h * N + nb + r) * K + c);
  }
  __syncthreads();
  if constexpr (kStageW) {
#pragma unroll
    for (int k = 0; k < kW; ++k) wf[k] = load8(sw + (16 * wave + col) * kStride + kq + 32 * k);
  }

  f32x4 acc[4] = {};
#pragma unroll
  for (int k = 0; k < kW; ++k) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[k], load8(sa + (16 * tt + col) * kStride + kq + 32 * k),
                                                        acc[tt], 0, 0, 0);
  }
  // acc[tt][i] = C[token t0 + 16 tt + col][column nb + 16 wave + 4 (lane >> 4) + i]
  const int n0 = nb + 16 * wave;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int t = t0 + 16 * tt + col;
    if (t < p.T) {
      uint16_t* dst = p.c + (size_t)t * p.c_t + (size_t)h * p.c_h + n0 + 4 * (lane >> 4);
      *(u32x2*)dst = u32x2{pack2(acc[tt][0], acc[tt][1]), pack2(acc[tt][2], acc[tt][3])};
    }
  }
  // The query's RoPE part is carried over unchanged (first column tile only).
  if (p.rope && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < kAbsorbTileT * (kDr / 8); i += kAbsorbThreads) {
      const int t = t0 + i / (kDr / 8);
      const int c8 = 8 * (i % (kDr / 8));
      if (t < p.T)
        *(uint4*)(p.c + (size_t)t * p.c_t + (size_t)h * p.c_h + N + c8) =
            *(const uint4*)(p.rope + ((size_t)t * p.H + h) * kDr + c8);
    }
  }
}

template __global__ void mla_absorb_kernel<kDh, 512>(AbsorbParams p);
template __global__ void mla_absorb_kernel<512, kDh>(AbsorbParams p);

}  // namespace mla
