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
//   * A workgroup (4 waves) owns 128 output columns and 64 tokens over a
//     slice of K: S slices per column tile (split K, S chosen on the host so
//     that the grid fills the chip), and within the workgroup each wave takes
//     a quarter of the slice, so no two waves load the same bytes.
//   * Wave tile: D^T[n][t] = W[n][:] . A[t][:] as 8 column tiles x 4 token
//     tiles of v_mfma_f32_16x16x32_bf16 (W rows as the A operand, token rows
//     as the B operand: both are 16-byte reads along K straight from memory
//     into registers), the next k step's 12 fragments in flight while this
//     one's 32 MFMAs run.
//   * The workgroups of one (column tile, K slice) that differ only in their
//     token chunk get consecutive ids on the same XCD, so W is fetched from
//     HBM once and found in that XCD's L2 by the others.
//   * End: the four waves' partial tiles are summed in LDS in a fixed order
//     (two halves of 64 columns); with S = 1 the workgroup writes bf16
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

constexpr int kRedStride = kOutProjTileN / 2 + 4;   // floats per LDS row of a half tile (padded)

}  // namespace

__global__ __launch_bounds__(kOutProjThreads, 2) void mla_outproj_kernel(OutProjParams p) {
  __shared__ __attribute__((aligned(16))) float red[4][kOutProjTileT][kRedStride];
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
  const int col = lane & 15;
  const int kq = 8 * (lane >> 4);
  const int n0 = nt * kOutProjTileN;
  const int t0 = tc * kOutProjTileT;
  const int kw = p.K / (p.splits * 4);                 // this wave's share of K
  const int kbeg = s * (p.K / p.splits) + wave * kw;

  // Fragment sources: W rows n0 + 16d + col, token rows t0 + 16r + col
  // (rows past T repeat row T-1; their outputs are never stored).
  const uint16_t* wsrc[8];
  const uint16_t* asrc[4];
#pragma unroll
  for (int d = 0; d < 8; ++d) wsrc[d] = p.w + (size_t)(n0 + 16 * d + col) * p.K + kbeg + kq;
#pragma unroll
  for (int r = 0; r < 4; ++r) asrc[r] = p.a + (size_t)min(t0 + 16 * r + col, p.T - 1) * p.K + kbeg + kq;

  f32x4 acc[8][4];
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[d][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wf[8], af[4];
#pragma unroll
  for (int d = 0; d < 8; ++d) wf[d] = load8(wsrc[d]);
#pragma unroll
  for (int r = 0; r < 4; ++r) af[r] = load8(asrc[r]);
  const int steps = kw / 32;
  for (int ks = 0; ks < steps; ++ks) {
    bf16x8 wn[8], an[4];
    const int nk = (ks + 1 < steps ? ks + 1 : ks) * 32;    // the last step reloads its own (unused) fragments
#pragma unroll
    for (int d = 0; d < 8; ++d) wn[d] = load8(wsrc[d] + nk);
#pragma unroll
    for (int r = 0; r < 4; ++r) an[r] = load8(asrc[r] + nk);
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[d][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[d], af[r], acc[d][r], 0, 0, 0);
#pragma unroll
    for (int d = 0; d < 8; ++d) wf[d] = wn[d];
#pragma unroll
    for (int r = 0; r < 4; ++r) af[r] = an[r];
  }

  // acc[d][r][i] = partial D^T[n0 + 16d + 4*(lane/16) + i][t0 + 16r + col].
  // Sum the four waves' partials in LDS, 64 columns at a time.
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(f32x4*)&red[wave][16 * r + col][16 * d + 4 * (lane >> 4)] = acc[4 * hf + d][r];
    __syncthreads();
    // Thread i sums 4 consecutive columns of one token row, 4 rows apart.
#pragma unroll
    for (int j = 0; j < (kOutProjTileT * kOutProjTileN / 2) / (4 * kOutProjThreads); ++j) {
      const int e = threadIdx.x + j * kOutProjThreads;       // index of a 4-column group
      const int t = e / (kOutProjTileN / 8);
      const int c4 = 4 * (e % (kOutProjTileN / 8));
      f32x4 v = *(const f32x4*)&red[0][t][c4];
      v += *(const f32x4*)&red[1][t][c4];
      v += *(const f32x4*)&red[2][t][c4];
      v += *(const f32x4*)&red[3][t][c4];
      const int tt = t0 + t;
      const int n = n0 + 64 * hf + c4;
      if (tt < p.T) {
        if (p.splits == 1)
          *(u32x2*)(p.out + (size_t)tt * p.N + n) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
        else
          *(f32x4*)(p.partial + ((size_t)s * p.T + tt) * p.N + n) = v;
      }
    }
    __syncthreads();
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
