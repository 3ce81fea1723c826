// Output projection over all heads (gfx950): u_t = W^O [o_{t,1}; ...; o_{t,n_h}].
//
// The second output equation of the MLA section of the deepseek.csdn.net
// FlashMLA article (section 2.2): the per-head outputs o_{t,i} (d_h = 128
// each, i.e. W^UV applied to the decode's latent output) are concatenated in
// head order and mapped by one matrix W^O [d_model][n_h * d_h].  With
// A = the concatenated rows [T][K] (K = n_h * 128, head-major: element
// (t, i * 128 + d) = o_{t,i}[d]) and W = W^O [N][K] (N = d_model):
//     out[t][n] = sum_k A[t][k] * W[n][k]
// bf16 in and out, fp32 accumulation.
//
// At decode sizes (tens to a few hundred tokens) W dominates the bytes
// (235 MB for d_model = 7168 and 128 heads) and every byte of it is used
// once per token, so the aim is to stream W from HBM exactly once while the
// token rows come from L2.  Work decomposition:
//   * A workgroup (8 waves) owns 128 output columns and 64 tokens over a
//     slice of K: S slices per column tile (split K, S chosen on the host so
//     that the grid fills the chip).  Wave w takes the column half w % 2
//     (64 columns) over the K quarter w / 2 of the slice, so no two waves
//     load the same weight bytes (the token rows, a few MB, come from L2).
//   * Wave tile: D^T[n][t] = W[n][:] . A[t][:] as 4 column tiles x 4 token
//     tiles of v_mfma_f32_16x16x32_bf16 (W rows as the A operand, token rows
//     as the B operand: both read along K straight from memory into
//     registers, 32 contiguous bytes per lane for two k steps, so a row's
//     128-byte line is read whole).  The stream is bound by how many bytes
//     are in flight, so every wave keeps the next pair of k steps' 16
//     fragments in flight while one pair's 32 MFMAs run: 16 KB per wave,
//     128 KB per compute unit.
//   * The workgroups of one (column tile, K slice) that differ only in their
//     token chunk get consecutive ids on the same XCD, so W is fetched from
//     HBM once and found in that XCD's L2 by the others.
//   * End: the four K quarters' partial tiles are summed in LDS in a fixed
//     order; with S = 1 the workgroup writes bf16
//     output, else fp32 partials that mla_outproj_reduce_kernel sums over the
//     S slices in slice order, so the result does not depend on scheduling.
#include <hip/hip_runtime.h>

#include "mla_outproj.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ inline bf16x8 load8(const uint16_t* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); }

constexpr int kKParts = kOutProjWaves / 2;           // K quarters per workgroup slice
constexpr int kRedStride = kOutProjTileN / 2 + 4;    // floats per LDS row of a column half (padded)

}  // namespace

__global__ __launch_bounds__(kOutProjThreads, 1) void mla_outproj_kernel(OutProjParams p) {
  __shared__ __attribute__((aligned(16))) float red[kOutProjWaves][kOutProjTileT][kRedStride];
  // Block -> (column tile, K slice, token chunk): the token chunks of one
  // (column tile, K slice) are consecutive blocks on one XCD.
  const int xcd = blockIdx.x % kNumXcdOutProj;
  const int k8 = blockIdx.x / kNumXcdOutProj;
  const int tc = k8 % p.tchunks;
  const int grp = (k8 / p.tchunks) * kNumXcdOutProj + xcd;
  if (grp >= p.ntiles * p.splits) return;
  const int nt = grp / p.splits;
  const int s = grp - nt * p.splits;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = wave & 1;                           // column half
  const int part = wave >> 1;                          // K quarter
  const int col = lane & 15;
  const int n0 = nt * kOutProjTileN + 64 * half;
  const int t0 = tc * kOutProjTileT;
  const int kw = p.K / (p.splits * kKParts);           // this wave's share of K (a multiple of 32)
  const int kbeg = s * (p.K / p.splits) + part * kw;

  // K goes in pairs of MFMA k steps (64 values): lane (col, g) loads the 16
  // values 64p + 16g .. +15 of its rows, 32 contiguous bytes, so the four
  // lanes of a row take one whole 128-byte line at once (read as two 64-byte
  // halves in different k steps, a line was often fetched twice), and hands
  // the first 8 to the MFMA of step 2p, the last 8 to step 2p + 1.  W and the
  // token rows use the same arrangement, so every MFMA still pairs equal k
  // and the sum over k is unchanged.  A wave's share with an odd number of
  // 32-value steps ends with one step in the plain arrangement (lane g takes
  // values 8g .. 8g + 7).  Rows past T repeat row T-1; their outputs are
  // never stored.
  const int g16 = 16 * (lane >> 4);
  const uint16_t* wsrc[4];
  const uint16_t* asrc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) wsrc[d] = p.w + (size_t)(n0 + 16 * d + col) * p.K + kbeg;
#pragma unroll
  for (int r = 0; r < 4; ++r) asrc[r] = p.a + (size_t)min(t0 + 16 * r + col, p.T - 1) * p.K + kbeg;

  f32x4 acc[4][4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[d][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One pair in flight ahead of the one being multiplied (16 KB per wave);
  // a pair past the wave's share reloads its last pair (in bounds, never
  // multiplied).
  const int steps = kw / 32;
  const int pairs = steps / 2;
  auto poff = [&](int pp) __attribute__((always_inline)) { return (pp < pairs ? pp : pairs - 1) * 64 + g16; };
  bf16x8 wf[2][2][4], af[2][2][4];   // [buffer][step of the pair][tile]
  auto load_pair = [&]<int B>(int pp) __attribute__((always_inline)) {
    const int o = poff(pp);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int d = 0; d < 4; ++d) wf[B][h][d] = load8(wsrc[d] + o + 8 * h);
#pragma unroll
      for (int r = 0; r < 4; ++r) af[B][h][r] = load8(asrc[r] + o + 8 * h);
    }
  };
  auto mma_pair = [&]<int B>() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[d][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[B][h][d], af[B][h][r], acc[d][r], 0, 0, 0);
  };
  // The scheduling barriers keep each pair's loads ahead of the other
  // buffer's MFMAs: left free, the compiler moves the loads down to just
  // before their own MFMAs (fewer live registers) and waits for them there,
  // so nothing is in flight during the MFMAs.
  if (pairs > 0) {
    load_pair.template operator()<0>(0);
    int pp = 0;
    for (; pp + 2 <= pairs; pp += 2) {
      load_pair.template operator()<1>(pp + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_pair.template operator()<0>();
      __builtin_amdgcn_sched_barrier(0);
      load_pair.template operator()<0>(pp + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma_pair.template operator()<1>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (pp < pairs) mma_pair.template operator()<0>();   // the last pair of an odd count, in buffer 0
  }
  if (steps & 1) {
    const int o = 64 * pairs + 8 * (lane >> 4);
    bf16x8 wt[4], at[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) wt[d] = load8(wsrc[d] + o);
#pragma unroll
    for (int r = 0; r < 4; ++r) at[r] = load8(asrc[r] + o);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[d][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wt[d], at[r], acc[d][r], 0, 0, 0);
  }

  // acc[d][r][i] = partial D^T[n0 + 16d + 4*(lane/16) + i][t0 + 16r + col].
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) *(f32x4*)&red[wave][16 * r + col][16 * d + 4 * (lane >> 4)] = acc[d][r];
  __syncthreads();
  // Thread i sums 4 consecutive columns of one token row over the K quarters
  // (waves half, half + 2, half + 4, half + 6), in that order.
#pragma unroll
  for (int j = 0; j < (kOutProjTileT * kOutProjTileN) / (4 * kOutProjThreads); ++j) {
    const int e = threadIdx.x + j * kOutProjThreads;    // 2048 groups: 64 rows x 128 columns / 4
    const int t = e / (kOutProjTileN / 4);
    const int c = 4 * (e % (kOutProjTileN / 4));         // column within the tile
    const int h = c / 64, c4 = c % 64;
    f32x4 v = *(const f32x4*)&red[h][t][c4];
#pragma unroll
    for (int q = 1; q < kKParts; ++q) v += *(const f32x4*)&red[h + 2 * q][t][c4];
    const int tt = t0 + t;
    const int n = nt * kOutProjTileN + c;
    if (tt < p.T) {
      if (p.splits == 1)
        *(u32x2*)(p.out + (size_t)tt * p.N + n) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      else
        *(f32x4*)(p.partial + ((size_t)s * p.T + tt) * p.N + n) = v;
    }
  }
}

// out[t][n] = bf16(sum over slices s = 0 .. S-1 of partial[s][t][n]), in slice order.
__global__ __launch_bounds__(256) void mla_outproj_reduce_kernel(OutProjParams p) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  const long long total = (long long)p.T * p.N;
  if (i >= total) return;
  f32x4 v = *(const f32x4*)(p.partial + i);
  for (int s = 1; s < p.splits; ++s) v += *(const f32x4*)(p.partial + (size_t)s * total + i);
  *(u32x2*)(p.out + i) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
}

}  // namespace mla
