// Device helpers shared by the two decode kernels (64-row and 128-row
// workgroups): LDS page layout and DMA staging, lane permutes for row
// reductions, and the worker's page cursor.
#pragma once

#include <utility>

#include "mla_kernels.h"

namespace mla {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kOverflowThreshold = 48.0f;   // log2 units: weights stay <= 2^48
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kBufferConfig = 0x00020000;   // buffer resource word 3 (raw, no swizzle)
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima),
// for waits on the kernel's own vector loads: issued through the builtin, the
// compiler knows they are complete after it.
constexpr int kWaitVmcnt0 = 0x0F70;

// Wait for the page DMAs, which the compiler does not see: in inline
// assembly, so that no pass can judge it redundant and drop it.
__device__ inline void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Pages of a sequence of `seqlen` tokens (0 for seqlen <= 0; no overflow
// near INT_MAX).
__device__ inline int pages_of(int seqlen) { return seqlen > 0 ? (seqlen - 1) / kPage + 1 : 0; }

// Read-only table entry at a wave-uniform address, through the constant
// address space: a scalar load, counted by lgkmcnt.  Keeping the kernel's own
// table reads off vmcnt means waiting for them never waits for page DMAs.
__device__ inline int32_t ld_uniform(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)ptr;
}

// LDS layout of a staged page: 72 tiles of 1 KB, tile (a, b) = rows 8a..8a+7 x
// 16-byte chunks 8b..8b+7 at byte (9a + b) * 1024; inside a tile, chunk c of
// row r sits at slot 8 * (r % 8) + ((c % 8) ^ (r % 8)).  The XOR spreads the
// rows a fragment read touches over distinct banks, and one wave-wide
// 16-byte DMA fills exactly one tile.
__device__ inline int lds_tile_offset(int r, int c) {
  return ((r >> 3) * 9 + (c >> 3)) * 1024 + ((r & 7) * 8 + ((c & 7) ^ (r & 7))) * 16;
}

// Stage one page of one latent head into LDS with 72 wave-wide DMAs, spread
// evenly over the waves, either at once (stage_page) or one at a time
// (stage_tile) among the previous page's MFMAs.  Lane u of the DMA for tile
// (a, b) fetches row 8a + u/8, chunk 8b + ((u%8) ^ (u/8)): a per-lane byte
// offset (lane_off) plus a wave-uniform one, relative to a buffer resource
// that spans exactly this page's 64 rows.
// All 64 rows are fetched; rows past the sequence end are zeroed afterwards by
// zero_tail_rows().
//
// The DMAs are issued from inline assembly (buffer_load_dwordx4 ... lds, with
// M0 holding the tile's LDS address), as composable_kernel does for gfx950:
// the compiler then does not know they write LDS and does not make the reads
// of the other buffer wait for them.  The kernel waits for them itself
// (s_waitcnt vmcnt(0) at the top of each page step) before any wave reads
// the buffer, and issues no vector load of its own between a DMA and that
// wait.  They write no registers.
__device__ inline __amdgpu_buffer_rsrc_t page_resource(const char* page_head, uint32_t page_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)page_head, (short)0, (int)page_bytes, (int)kBufferConfig);
}

// Buffer resource over page `pid` of the latent head whose first row starts
// at kv_head.  A page id outside [0, num_pages) (a bad block_table entry)
// gets a resource of size 0: its DMAs then read zeros and no address outside
// the cache is ever formed.
__device__ inline __amdgpu_buffer_rsrc_t page_rsrc(const char* kv_head, int pid, int num_pages, size_t page_stride,
                                                   uint32_t page_bytes) {
  const bool ok = (unsigned)pid < (unsigned)num_pages;
  return page_resource(kv_head + (ok ? (size_t)pid * page_stride : (size_t)0), ok ? page_bytes : 0u);
}

// One wave-wide DMA: lane u reads 16 bytes at the resource's base +
// lane_off(u) + soff, and LDS receives them at m0 + 16u.
__device__ inline void lds_dma16(uint32_t m0, uint32_t lane_off, __amdgpu_buffer_rsrc_t rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(lane_off), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// The same DMA with compile-time offsets: LDS at m0_base + kLds, source at
// soff + kSrc.  The instruction's offset field adds kSrc to the source and
// to the LDS address alike, so M0 is set to m0_base + kLds - kSrc by one
// scalar add; the tiles of one tile row (source 128 bytes apart, LDS 1 KB
// apart) then share one base and one source offset register.
template <int kLds, int kSrc>
__device__ inline void lds_dma16_at(uint32_t m0_base, uint32_t lane_off, __amdgpu_buffer_rsrc_t rsrc, uint32_t soff) {
  static_assert(kSrc >= 0 && kSrc < 4096 && kLds >= kSrc, "12-bit offset field; M0 at or above the base");
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen offset:%5 lds"
               :
               : "s"(m0_base), "v"(lane_off), "s"(rsrc), "s"(soff), "i"(kLds - kSrc), "i"(kSrc)
               : "memory", "m0", "scc");
}

// DMA number k (0 .. kPerWave-1) of this wave for one page, when each of the
// workgroup's waves issues kPerWave of the page's 72: tile j = kPerWave *
// wave + k, i.e. tile row j / 9 (rows 8*(j/9) ..+7) x tile column j % 9
// (chunks 8*(j%9) ..+7).  m0_wave is the LDS address of the wave's first
// tile (the page buffer + kPerWave KB per wave) and soff_rows[r] the source
// offset of its tile row r (8 rows per tile row); the tile column is a
// compile-time offset.
template <int kPerWave>
struct WaveTiles {
  static_assert(kPerWave % 9 == 0 && (kPageBytes / 1024) % kPerWave == 0, "whole tile rows per wave");
  uint32_t soff_rows[kPerWave / 9];
  __device__ WaveTiles(int wave, int row_stride_bytes) {
#pragma unroll
    for (int r = 0; r < kPerWave / 9; ++r) soff_rows[r] = (uint32_t)((wave * (kPerWave / 9) + r) * 8 * row_stride_bytes);
  }
};

template <int kPerWave, int k>
__device__ inline void stage_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, uint32_t m0_wave,
                                  const WaveTiles<kPerWave>& t) {
  lds_dma16_at<k * 1024, (k % 9) * 128>(m0_wave, lane_off, rsrc, t.soff_rows[k / 9]);
}

template <int kPerWave>
__device__ inline void stage_page(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, uint32_t m0_wave,
                                  const WaveTiles<kPerWave>& t) {
  [&]<int... k>(std::integer_sequence<int, k...>) __attribute__((always_inline)) {
    (stage_tile<kPerWave, k>(rsrc, lane_off, m0_wave, t), ...);
  }(std::make_integer_sequence<int, kPerWave>{});
}

// Zero rows [valid, 64) of a staged page (its cache slots lie past the
// sequence end and may hold anything, NaN included); kThreadsIn threads.
template <int kThreadsIn>
__device__ inline void zero_tail_rows(char* page, int valid, int tid) {
  for (int i = valid * kChunksPerRow + tid; i < kPageChunks; i += kThreadsIn) {
    const int r = i / kChunksPerRow;
    const int c = i - r * kChunksPerRow;
    *(u32x4*)(page + lds_tile_offset(r, c)) = u32x4{0, 0, 0, 0};
  }
}

// The 4 lanes l, l^16, l^32, l^48 hold the same query row.  With both
// operands equal to x, v_permlane16_swap leaves {x[l], x[l^16]} in lane l's
// pair of results and v_permlane32_swap {x[l], x[l^32]}; a symmetric
// reduction of the pair is the xor-shuffle step, without an LDS round trip
// (which would also wait for the fragment reads in flight).
__device__ inline float xor16_pair(float x, bool max_op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  const float a = __builtin_bit_cast(float, (uint32_t)r[0]), b = __builtin_bit_cast(float, (uint32_t)r[1]);
  return max_op ? fmaxf(a, b) : a + b;
}
__device__ inline float xor32_pair(float x, bool max_op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  const float a = __builtin_bit_cast(float, (uint32_t)r[0]), b = __builtin_bit_cast(float, (uint32_t)r[1]);
  return max_op ? fmaxf(a, b) : a + b;
}
__device__ inline float row_max4(float x) { return xor32_pair(xor16_pair(x, true), true); }

// Larger of two scores.  NaN-propagating maximum (v_maximum3_f32): unlike
// fmaxf it needs no quieting of its inputs first.  Scores are never NaN
// (slots past a sequence's end are zeroed in LDS before use).
__device__ inline float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float row_sum4(float x) { return xor32_pair(xor16_pair(x, false), false); }

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// acc + the two bf16 values packed by pack_bf16x2, in fp32: one
// v_dot2c_f32_bf16 against (1, 1) (on this chip vector ALU cycles add to
// the matrix core's, so the sum takes one instruction, not four).  Each row
// keeps two sums: the exact one, for its log-sum-exp, and one over the
// rounded weights that the PV product actually uses, which normalises O, so
// that each output row is a convex combination of cached values: the
// rounding of a weight then moves O only by that weight's share of
// (v_j - O), never by a mismatch between the weights and their sum.
__device__ inline float add_bf16x2(float acc, uint32_t packed) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                          acc, false);
}

// Physical page of logical block j of sequence b.  A block past the end of
// the table row (a length above 64 * max_pages) reads as -1, never as the
// next row or past the table.
__device__ inline int page_id(const DecodeParams& p, int b, int j) {
  return j < p.max_pages ? ld_uniform(p.block_table + (size_t)b * p.max_pages + j) : -1;
}

// End page of sequence b's part of this worker's range.
__device__ inline int segment_end(const int32_t* meta, const int32_t* seqlens, int b) {
  return b == ld_uniform(meta + 2) ? ld_uniform(meta + 3) : pages_of(ld_uniform(seqlens + b));
}

// Advance (b, page, end) to the worker's next page; returns false past the
// end.  p0 is the first page of the cursor's segment (0 on entering a new
// sequence).
__device__ inline bool next_page(const int32_t* meta, const int32_t* seqlens, int& b, int& page, int& end, int& p0) {
  if (++page < end) return true;
  for (int nb = b + 1; nb <= ld_uniform(meta + 2); ++nb) {
    const int e = segment_end(meta, seqlens, nb);
    if (e > 0) {
      b = nb;
      page = 0;
      end = e;
      p0 = 0;
      return true;
    }
  }
  return false;
}

// Page that step `page` of segment [p0, end) processes, in row block rb of
// nrb.  The row blocks of a head read the same pages, and a page's fetch
// takes its full memory latency while its twins in the other blocks are in
// flight for the same page.  So after the segment's first page (whose maxima
// set the softmax references, first in every block), pages go in groups of
// nrb, and block rb takes a group's pages rotated by rb: at each group step
// every block fetches a different page, and a page is fetched from memory by
// one block and found in L2 by the others.  A last, partial group keeps its
// order.  The result does not otherwise depend on the order.
// Two row blocks (128 query rows per latent head) are the common case and
// take shifts and masks instead of a division.
__device__ inline int page_in_order(int page, int p0, int end, int rb, int nrb) {
  const int j = page - p0 - 1;
  if (j < 0 || nrb == 1) return page;
  if (nrb == 2) {
    const int base = p0 + 1 + (j & ~1);
    if (base + 2 > end) return page;
    return base + ((j & 1) ^ rb);
  }
  const int base = p0 + 1 + (j / nrb) * nrb;
  if (base + nrb > end) return page;
  const int r = j - (j / nrb) * nrb + rb;
  return base + (r >= nrb ? r - nrb : r);
}

}  // namespace dev
}  // namespace mla
