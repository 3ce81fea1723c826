// Split-KV paged MLA decode kernel for gfx950 (MI355X).
//
// What it computes: the MLA output equation of the deepseek.csdn.net FlashMLA
// article (section 2.2) after matrix absorption -- each absorbed query row
// (576 wide) attends over the sequence's cached latent rows [c^KV; k^R] and
// sums their first 512 columns (c^KV) with the softmax weights -- over one
// split of the paged cache (section 4.2(1): 64-token pages found through
// block_table, a split-KV forward kernel, then a combine kernel).
//
// Work decomposition (MI355X-native):
//   * One workgroup = 4 waves = 64 query rows of one latent head, over the
//     page range the scheduler gave its worker.  The workgroups that serve
//     the other row blocks of the same head read the same pages; they are
//     dispatched back to back on the same XCD so the second read hits L2.
//   * Wave v owns query rows 16v..16v+15.  Its absorbed Q (16 x 576 bf16) sits
//     in VGPRs as MFMA B fragments for the whole segment; its output
//     O^T (512 x 16 fp32) sits in 32 v_mfma_f32_16x16x32_bf16 accumulators
//     (128 accumulation registers).
//   * A page is processed as two k-steps of 32 keys.  Per k-step: S^T = K Q^T
//     for two 16-key tiles (A = K rows from LDS, B = Q), the softmax weights
//     in the accumulator layout (each lane holds 4 keys of one query row),
//     then O^T += V^T P^T (A = V columns read with the transposing
//     ds_read_b64_tr_b16, B = P taken straight from the S^T accumulators).
//   * Pages move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging; the buffer resource bounds every read to the page), double
//     buffered: page i+1 is in flight while page i is computed.  The page
//     sits in LDS as 72 tiles of 1 KB (8 rows x 8 chunks of 16 bytes) with the
//     16-byte chunks XOR-swizzled by row inside a tile.
//   * Softmax runs in base 2 with the scale folded into one multiply.  Each
//     row keeps a reference point m (its maximum over the segment's first
//     k-step) and accumulates unnormalised weights 2^(s - m) <= 2^48; that is
//     exact math, and bf16/fp32 have the range for it (sums stay below 2^65
//     times the largest cached value for 2^17 keys).  The output tile is
//     therefore never rescaled: only MFMAs touch it, which keeps it in the
//     accumulation registers with no copies.  Should a later k-step exceed a
//     row's reference by more than 48, the segment is void: the workgroup
//     records it, with every row's maximum over the segment, and a second
//     launch of one workgroup recomputes it with those maxima as references,
//     where no weight exceeds 1.  For attention scores of any ordinary spread
//     nothing is recorded and the second launch only scans the flags.
//   * Keys a query may not see (tail slots of the last page, causal future)
//     get weight 0, and tail rows of the last page are zeroed in LDS so that
//     whatever the cache holds there never reaches O.
#include <utility>

#include "mla_kernels.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kOverflowThreshold = 48.0f;   // log2 units: weights stay <= 2^48
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kBufferConfig = 0x00020000;   // buffer resource word 3 (raw, no swizzle)
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima).
// Issued through the builtin, the compiler knows every vector memory
// operation -- its own and the page DMAs -- is complete after it.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ inline int pages_of(int seqlen) { return (seqlen + kPage - 1) / kPage; }

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

// Stage one page of one latent head into LDS with 72 wave-wide DMAs (18 per
// wave), either at once (stage_page) or one at a time (stage_tile) spread
// through the previous page's MFMAs.  Lane u of the DMA for tile (a, b) fetches row 8a + u/8, chunk
// 8b + ((u%8) ^ (u/8)): a per-lane byte offset (lane_off) plus a wave-uniform
// one, relative to a buffer resource that spans exactly this page's 64 rows.
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

// DMA number k (0 .. kLdsDmaPerWave-1) of this wave for one page: tile
// j = 4k + wave, i.e. rows 8a..8a+7 x chunks 8b..8b+7 with j = 9a + b.
__device__ inline void stage_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, int row_stride_bytes,
                                  uint32_t lds_dst, int wave, int k) {
  const int j = k * kWaves + wave;            // tile index 9a + b, wave-uniform
  const int a = j / 9, b = j - (j / 9) * 9;
  const uint32_t m0 = lds_dst + j * 1024;
  const uint32_t soff = a * 8 * row_stride_bytes + b * 128;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(lane_off), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ inline void stage_page(const char* page_head, uint32_t page_bytes, uint32_t lane_off,
                                  int row_stride_bytes, uint32_t lds_dst, int wave) {
  const __amdgpu_buffer_rsrc_t rsrc = page_resource(page_head, page_bytes);
#pragma unroll
  for (int k = 0; k < kLdsDmaPerWave; ++k) stage_tile(rsrc, lane_off, row_stride_bytes, lds_dst, wave, k);
}

// Zero rows [valid, 64) of a staged page (its cache slots lie past the
// sequence end and may hold anything, NaN included).
__device__ inline void zero_tail_rows(char* page, int valid, int tid) {
  for (int i = valid * kChunksPerRow + tid; i < kPageChunks; i += kThreads) {
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
__device__ inline float row_sum4(float x) { return xor32_pair(xor16_pair(x, false), false); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// End page of sequence b's part of this worker's range.
__device__ inline int segment_end(const int32_t* meta, const int32_t* seqlens, int b) {
  return b == ld_uniform(meta + 2) ? ld_uniform(meta + 3) : pages_of(ld_uniform(seqlens + b));
}

// Advance (b, page, end) to the worker's next page; returns false past the end.
__device__ inline bool next_page(const int32_t* meta, const int32_t* seqlens, int& b, int& page, int& end) {
  if (++page < end) return true;
  for (int nb = b + 1; nb <= ld_uniform(meta + 2); ++nb) {
    const int e = segment_end(meta, seqlens, nb);
    if (e > 0) {
      b = nb;
      page = 0;
      end = e;
      return true;
    }
  }
  return false;
}

}  // namespace

// One worker's pages for latent head g and row block rb: every segment in the
// worker's range [meta[0], meta[1]) .. [meta[2], meta[3]).
//
// kSingleHead: h_kv == 1, so a page's rows are contiguous 1152-byte rows and
// every stride is a compile-time constant.
// kRedo: the worker is one segment that overflowed in the first launch
// (meta is its redo record); each row starts from the reference point
// recorded for it, which is its maximum score over the segment.
template <bool kSingleHead, bool kRedo>
__device__ __forceinline__ void decode_worker(const DecodeParams& p, char (*lds_page)[kPageBytes],
                                              const int32_t* meta, int g, int rb, int redo_item) {
  const uint32_t lds_base = (uint32_t)(uintptr_t)&lds_page[0][0];   // LDS byte address
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp4 = lane >> 4;     // which 4-key / 8-wide k slice of an MFMA fragment
  const int col = lane & 15;      // query row within the wave's tile / MFMA column

  const int meta_b0 = ld_uniform(meta + 0), meta_b1 = ld_uniform(meta + 2);
  if (meta_b1 < meta_b0) return;                       // worker without pages
  // Compute cursor (cb, cpage, cend) and load cursor (lb, lpage, lend).
  int cb = meta_b0, cpage = ld_uniform(meta + 1), cend = segment_end(meta, p.seqlens, cb);
  if (cpage >= cend) return;
  int lb = cb, lpage = cpage, lend = cend;
  bool lvalid = true;

  const int row_stride_bytes = kSingleHead ? kRowBytes : p.h_kv * kRowBytes;   // bytes between tokens
  const size_t page_stride_bytes = (size_t)kPage * row_stride_bytes;
  const uint32_t page_span = (uint32_t)(kPage * row_stride_bytes);              // resource size
  const char* kv_head = (const char*)p.kv + (size_t)g * kRowBytes;
  const uint32_t lane_src_off = (lane >> 3) * row_stride_bytes + ((lane & 7) ^ (lane >> 3)) * 16;

  // This lane's query row.
  const int qrow = rb * kRowsPerBlock + wave * kRowsPerWave + col;
  const bool row_ok = qrow < p.rows;
  const int q_tok = row_ok ? qrow / p.group : 0;
  const int q_head = g * p.group + (row_ok ? qrow - q_tok * p.group : 0);

  // First page in flight before anything else; the id of the page after it
  // is read now, one page ahead of its DMAs.
  int next_pid = 0;
  {
    const int page_id = ld_uniform(p.block_table + (size_t)lb * p.max_pages + lpage);
    lvalid = next_page(meta, p.seqlens, lb, lpage, lend);
    stage_page(kv_head + (size_t)page_id * page_stride_bytes, page_span, lane_src_off, row_stride_bytes,
               lds_base, wave);
    if (lvalid) next_pid = ld_uniform(p.block_table + (size_t)lb * p.max_pages + lpage);
  }

  int it = 0;
  while (true) {
    // ---------------- segment: pages [cpage, cend) of sequence cb ----------------
    const int b = cb;
    const int L = ld_uniform(p.seqlens + b);
    const int s0 = ld_uniform(p.num_splits + b);
    const int nsplit = ld_uniform(p.num_splits + b + 1) - s0;
    const int slot = s0 + (b == meta_b0 ? ld_uniform(meta + 4) : 0);
    const int n_vis_row = p.causal ? L - p.s_q + q_tok + 1 : L;
    const int seg_page0 = cpage;

    // Q fragments: lane (col, grp4) holds row qrow, dims 32*ks + 8*grp4 .. +7.
    bf16x8 qf[kDqk / 32];
    {
      const uint16_t* qp = p.q + ((size_t)(b * p.s_q + q_tok) * p.h_q + q_head) * kDqk + grp4 * 8;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        u32x4 v = row_ok ? *(const u32x4*)(qp + ks * 32) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    float m_ref = kNegInf;      // this row's reference point (log2 units)
    if constexpr (kRedo) m_ref = p.redo_m[(size_t)redo_item * kRowsPerBlock + wave * kRowsPerWave + col];
    float m_seen = kNegInf;     // largest score seen in the segment
    float l_run = 0.f;          // this lane's share of sum_j 2^(s_j - m_ref)
    int overflow = 0;           // this lane's row outgrew its reference
    f32x4 acc[kDv / 16];

    // One pass over the segment's pages.  The output tiles are zeroed here
    // and only MFMAs touch them until the segment epilogue.  The page
    // prefetched for the next segment (if any) is waited for at the top of
    // that segment's first page step.
    auto pass = [&]() __attribute__((always_inline)) {
      // Zero from an MFMA, so that the tiles are born in the accumulation
      // registers rather than copied there from VGPRs on every page.
      const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      const f32x4 zero4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zero8, zero8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < kDv / 16; ++nt) acc[nt] = zero4;
      l_run = 0.f;
      // The loop leaves at its bottom, so the tiles' loop-carried value has
      // the next page's first MFMA as its only use and every MFMA can
      // accumulate in place.
      while (true) {
        // Page `it` has landed in every wave's share and the buffer of page
        // it-1 is free.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        char* buf = lds_page[it & 1];
        const int valid = min(kPage, L - cpage * kPage);
        if (valid < kPage) {
          zero_tail_rows(buf, valid, tid);
          __syncthreads();
        }
        // The next page's DMAs go out one by one inside this page's MFMA
        // stream (below); its id was read a page ago.  The cursor moves on
        // and the id after it is read now.
        const bool dma = lvalid;
        const __amdgpu_buffer_rsrc_t dma_rsrc =
            page_resource(kv_head + (size_t)next_pid * page_stride_bytes, page_span);
        const uint32_t dma_dst = lds_base + ((it + 1) & 1) * kPageBytes;
        if (lvalid) {
          lvalid = next_page(meta, p.seqlens, lb, lpage, lend);
          if (lvalid) next_pid = ld_uniform(p.block_table + (size_t)lb * p.max_pages + lpage);
        }

        // Per-lane LDS bases of this page's fragment reads; every read is one
        // of them plus a compile-time offset below 64 KB.  They are formed
        // here from the lane id rather than kept live across the loop, and the
        // empty asm statements stop the compiler from hoisting them or turning
        // base + offset into an OR that the DS immediate offset cannot absorb.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t page_base = (uint32_t)(uintptr_t)buf;
        uint32_t kb[2], vb[4];
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          // K row (ln & 15) (+16 per key tile), chunk 4*par + (ln >> 4) (+8 per 2 k-steps)
          kb[par] = page_base + lds_tile_offset(ln & 15, 4 * par + (ln >> 4));
          asm volatile("" : "+v"(kb[par]));
        }
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          // V row (ln >> 2) (+16 per read), columns 16*m4 + 4*(ln & 3) (+64 per 4 tiles)
          vb[m4] = page_base + lds_tile_offset(ln >> 2, 2 * m4 + ((ln & 3) >> 1)) + 8 * (ln & 1);
          asm volatile("" : "+v"(vb[m4]));
        }

        const int key0 = cpage * kPage;

        // Fragment reads.  K: lane (col, grp4) of read i = 2*ks + tt of
        // k-step kk holds key 32kk + 16tt + col, chunk 4*ks + grp4 (the A
        // operand of S^T = K Q^T).  V: the A operand of O^T += V^T P^T for
        // column tile nt needs, in lane (n = col, grp4), V[key][16nt + n] for
        // keys 32kk + 4*grp4 + m and 32kk + 16 + 4*grp4 + m: two transposing
        // reads of 4 rows x 16 columns, where lane l fetches row l/4,
        // columns 4*(l%4)..+3 of the 16-column tile.
        auto read_k = [&](int kk, int i) __attribute__((always_inline)) {
          const int ks = i >> 1, tt = i & 1;
          return *(lds_bf16x8*)(kb[ks & 1] + (uint32_t)((2 * (2 * kk + tt) * 9 + (ks >> 1)) * 1024));
        };
        auto read_v = [&](int kk, int nt) __attribute__((always_inline)) {
          const uint32_t o0 = (uint32_t)(((4 * kk + 0) * 9 + (nt >> 2)) * 1024);
          const uint32_t o1 = (uint32_t)(((4 * kk + 2) * 9 + (nt >> 2)) * 1024);
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb[nt & 3] + o0));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb[nt & 3] + o1));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };

        // Softmax weights (base 2) of k-step kk in eight short stages, each
        // placed between two MFMAs of the stream so that its VALU work and
        // latency hide behind the matrix pipe.  Lane (col, grp4) holds, for
        // its query row, key key0 + 32kk + 16tt + 4*grp4 + i in s[kk][tt][i];
        // keys the row may not see get weight 0 (no branch: every page masks).
        f32x4 s[2][2];
        float x[2][8], rm[2], mu[2], w[2][8];
        bf16x8 pf[2];
        auto softmax_stage = [&](int kk, int st) __attribute__((always_inline)) {
          if (st == 0) {
            float r = kNegInf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = key0 + 32 * kk + 16 * (e >> 2) + 4 * grp4 + (e & 3);
              const float v = s[kk][e >> 2][e & 3] * p.scale_log2;
              x[kk][e] = key < n_vis_row ? v : kNegInf;
              r = fmaxf(r, x[kk][e]);
            }
            rm[kk] = r;
          } else if (st == 1) {
            rm[kk] = xor16_pair(rm[kk], true);
          } else if (st == 2) {
            const float r = xor32_pair(rm[kk], true);
            m_seen = fmaxf(m_seen, r);
            if (m_ref == kNegInf) {
              m_ref = r;            // nothing accumulated yet: adopt this maximum
            } else if (r > m_ref + kOverflowThreshold) {
              overflow = 1;         // this segment's result for the row is void
            }
            mu[kk] = m_ref == kNegInf ? 0.f : m_ref;
          } else if (st < 7) {
            const int e = 2 * (st - 3);
            w[kk][e] = __builtin_amdgcn_exp2f(x[kk][e] - mu[kk]);
            w[kk][e + 1] = __builtin_amdgcn_exp2f(x[kk][e + 1] - mu[kk]);
            l_run += w[kk][e] + w[kk][e + 1];
          } else {
            // B operand of the output MFMA: slot e holds key 16*(e/4) + 4*grp4 + e%4.
            pf[kk] = __builtin_bit_cast(
                bf16x8, u32x4{pack_bf16x2(w[kk][0], w[kk][1]), pack_bf16x2(w[kk][2], w[kk][3]),
                              pack_bf16x2(w[kk][4], w[kk][5]), pack_bf16x2(w[kk][6], w[kk][7])});
          }
        };

        // The page's instruction stream, in issue order: 72 score MFMAs (two
        // k-steps, two interleaved chains each) then 64 output MFMAs.  After
        // MFMA g come: the K read kKAhead MFMAs ahead, the V read kVAhead
        // output MFMAs ahead, every kDmaEvery-th MFMA one DMA of the next
        // page, and the softmax stages of k-step 0 (during the k-step 1
        // scores) and of k-step 1 (during the k-step 0 outputs).
        // sched_barrier(0) pins that order.
        constexpr int kKReads = 2 * (kDqk / 32);   // 36 score MFMAs per k-step
        constexpr int kQk = 2 * kKReads;           // 72
        constexpr int kPv = 2 * (kDv / 16);        // 64
        constexpr int kKAhead = 8;
        constexpr int kVAhead = 4;
        constexpr int kDmaEvery = 5;
        constexpr int kSm0At = kKReads + 1;        // first stage of k-step 0's softmax
        constexpr int kSm1At = kQk + 1;            // first stage of k-step 1's softmax
        constexpr int kSmEvery = 3;
        static_assert(kSm0At + 7 * kSmEvery < kQk, "k-step 0 weights ready before its outputs");
        static_assert(kSm1At + 7 * kSmEvery < kQk + kPv / 2, "k-step 1 weights ready before its outputs");
        static_assert(kDmaEvery * kLdsDmaPerWave <= kQk + kPv, "every DMA inside the stream");
        bf16x8 kf[kQk];
        bf16x8 vf[kPv];
#pragma unroll
        for (int i = 0; i < kKAhead; ++i) kf[i] = read_k(i / kKReads, i % kKReads);
        __builtin_amdgcn_sched_barrier(0);
        // One step of the stream; G is a template parameter so that every
        // array index and schedule decision is a compile-time constant.
        auto step = [&]<int G>() __attribute__((always_inline)) {
          constexpr int g = G;
          if constexpr (g < kQk) {
            constexpr int kk = g / kKReads, i = g % kKReads;
            const f32x4 c = i < 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kk][i & 1];
            s[kk][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[g], qf[i >> 1], c, 0, 0, 0);
          } else {
            constexpr int n = g - kQk, kk = n / (kPv / 2), nt = n % (kPv / 2);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n], pf[kk], acc[nt], 0, 0, 0);
          }
          if constexpr (g + kKAhead < kQk) kf[g + kKAhead] = read_k((g + kKAhead) / kKReads, (g + kKAhead) % kKReads);
          {
            constexpr int v = g + kVAhead - kQk;   // V read issued after MFMA g
            if constexpr (v >= 0 && v < kPv) vf[v] = read_v(v / (kPv / 2), v % (kPv / 2));
          }
          if constexpr (g % kDmaEvery == 0 && g / kDmaEvery < kLdsDmaPerWave) {
            if (dma) stage_tile(dma_rsrc, lane_src_off, row_stride_bytes, dma_dst, wave, g / kDmaEvery);
          }
          if constexpr (g >= kSm0At && (g - kSm0At) % kSmEvery == 0 && (g - kSm0At) / kSmEvery < 8)
            softmax_stage(0, (g - kSm0At) / kSmEvery);
          if constexpr (g >= kSm1At && (g - kSm1At) % kSmEvery == 0 && (g - kSm1At) / kSmEvery < 8)
            softmax_stage(1, (g - kSm1At) / kSmEvery);
          __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... G>(std::integer_sequence<int, G...>) __attribute__((always_inline)) {
          (step.template operator()<G>(), ...);
        }(std::make_integer_sequence<int, kQk + kPv>{});

        ++it;
        if (cpage + 1 == cend) break;
        ++cpage;
      }
    };

    pass();
    bool write_out = row_ok;
    if constexpr (!kRedo) {
      // A segment where some row overflowed is recorded for the redo launch
      // (with every row's maximum) and leaves its outputs to it.  Every
      // segment writes its flag, so stale flags never survive a call.
      const int item = (slot * p.h_kv + g) * p.row_blocks + rb;
      const int ovf = __syncthreads_or(overflow);
      if (tid == 0) p.redo_flag[item] = ovf;
      if (ovf) {
        if (tid < kMetaInts) {
          const int rec[kMetaInts] = {b, seg_page0, b, cend, slot - s0, 0, 0, 0};
          p.redo_meta[(size_t)item * kMetaInts + tid] = rec[tid];
        }
        if (grp4 == 0) p.redo_m[(size_t)item * kRowsPerBlock + wave * kRowsPerWave + col] = m_seen;
        write_out = false;
      }
    }

    // ---------------- segment epilogue ----------------
    const float l_tot = row_sum4(l_run);
    const bool empty = l_tot == 0.f;
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_nat = empty ? kNegInf : (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
    // Lane (col, grp4) holds O[qrow][16*nt + 4*grp4 + i] in acc[nt][i].
    if (write_out) {
      if (nsplit == 1) {
        uint16_t* op = p.o + ((size_t)(b * p.s_q + q_tok) * p.h_q + q_head) * kDv + 4 * grp4;
#pragma unroll
        for (int nt = 0; nt < kDv / 16; ++nt) {
          uint2 v;
          v.x = pack_bf16x2(acc[nt][0] * inv, acc[nt][1] * inv);
          v.y = pack_bf16x2(acc[nt][2] * inv, acc[nt][3] * inv);
          *(uint2*)(op + 16 * nt) = v;
        }
        if (grp4 == 0) p.lse[((size_t)b * p.h_q + q_head) * p.s_q + q_tok] = lse_nat;
      } else {
        float* wp = p.ws_o + ((size_t)(slot * p.h_kv + g) * p.rows + qrow) * kDv + 4 * grp4;
#pragma unroll
        for (int nt = 0; nt < kDv / 16; ++nt) *(f32x4*)(wp + 16 * nt) = acc[nt] * inv;
        if (grp4 == 0) p.ws_lse[(size_t)(slot * p.h_kv + g) * p.rows + qrow] = lse_nat;
      }
    }

    // Next segment: the sequence after this one in the worker's range.
    if (cb == meta_b1) break;
    int nb = cb, np = cpage, ne = cend;
    if (!next_page(meta, p.seqlens, nb, np, ne)) break;
    cb = nb;
    cpage = np;
    cend = ne;
  }
}

template <bool kSingleHead>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_page[2][kPageBytes];
  // Block -> (worker, latent head, row block).  Blocks are dispatched to the
  // XCDs round-robin; the row blocks of one (worker, head) share its KV
  // stream, so they are given ids on the same XCD, issued back to back.
  const int xcd = blockIdx.x % kNumXcd;
  const int k = blockIdx.x / kNumXcd;
  const int rb = k % p.row_blocks;
  const int grp = (k / p.row_blocks) * kNumXcd + xcd;
  if (grp >= p.num_workers * p.h_kv) return;
  const int worker = grp / p.h_kv;
  const int g = grp - worker * p.h_kv;
  decode_worker<kSingleHead, false>(p, lds_page, p.meta + (size_t)worker * kMetaInts, g, rb, -1);
}

// One workgroup redoes, one after another, the segments the decode launch
// flagged (none for ordinary scores: the launch then only scans the flags).
template <bool kSingleHead>
__global__ __launch_bounds__(kThreads, 1) void mla_redo_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_page[2][kPageBytes];
  __shared__ int list[kRedoScan];
  __shared__ int n_list;
  const int tid = threadIdx.x;
  const int total = p.num_splits[p.batch] * p.h_kv * p.row_blocks;
  for (int base = 0; base < total; base += kRedoScan) {
    if (tid == 0) n_list = 0;
    __syncthreads();
    for (int i = base + tid; i < min(total, base + kRedoScan); i += kThreads)
      if (p.redo_flag[i]) list[atomicAdd(&n_list, 1)] = i;
    __syncthreads();
    const int n = n_list;
    for (int e = 0; e < n; ++e) {
      const int item = list[e];
      const int rb = item % p.row_blocks;
      const int g = (item / p.row_blocks) % p.h_kv;
      decode_worker<kSingleHead, true>(p, lds_page, p.redo_meta + (size_t)item * kMetaInts, g, rb, item);
      __syncthreads();
    }
  }
}

template __global__ void mla_decode_kernel<true>(DecodeParams p);
template __global__ void mla_decode_kernel<false>(DecodeParams p);
template __global__ void mla_redo_kernel<true>(DecodeParams p);
template __global__ void mla_redo_kernel<false>(DecodeParams p);

}  // namespace mla
