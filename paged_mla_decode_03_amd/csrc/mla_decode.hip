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
//   * One workgroup = 8 waves (two per SIMD) = 64 query rows of one latent
//     head, over the page range the scheduler gave its worker.  The
//     workgroups that serve the other row blocks of the same head read the
//     same pages; they are dispatched back to back on the same XCD so the
//     second read hits L2.
//   * Scores: wave v takes score row tile v % 4 (16 query rows) against key
//     half v / 4 (32 keys) of a page.  Its absorbed Q (16 x 576 bf16) sits in
//     VGPRs as MFMA B fragments for the whole segment; S^T = K Q^T is 2 key
//     tiles x 18 k-steps of v_mfma_f32_16x16x32_bf16 with K fragments read
//     from LDS.
//   * Softmax in the score accumulators' layout (each lane holds 4 keys of
//     one row per tile), row maxima and sums with lane permutes and, across
//     the two key halves, through LDS; the bf16 weights P go to LDS.
//   * Outputs: wave v owns output columns 64v..64v+63 for all 64 rows,
//     O^T += V^T P^T (A = V columns read with the transposing
//     ds_read_b64_tr_b16, B = P from LDS), 16 accumulators (64 registers)
//     that only MFMAs touch.  With two waves per SIMD, one wave's softmax,
//     LDS waits and DMA issue overlap the other's MFMAs.
//   * Pages move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging; the buffer resource bounds every read to the page), double
//     buffered: page i+1's 72 DMAs go out one by one between page i's MFMAs.
//     The page sits in LDS as 72 tiles of 1 KB (8 rows x 8 chunks of 16
//     bytes) with the 16-byte chunks XOR-swizzled by row inside a tile.
//   * Softmax runs in base 2 with the scale folded into one multiply.  Each
//     row keeps a reference point m (its maximum over the segment's first
//     page) and accumulates unnormalised weights 2^(s - m) <= 2^48; that is
//     exact math, and bf16/fp32 have the range for it (sums stay below 2^65
//     times the largest cached value for 2^17 keys).  The output tile is
//     therefore never rescaled.  Should a later page exceed a row's
//     reference by more than 48, the pass is void and the workgroup runs the
//     segment again with each row's maximum over the segment as its
//     reference, where no weight exceeds 1.  For attention scores of any
//     ordinary spread the second pass never runs.
//   * Keys a query may not see (tail slots of the last page, causal future)
//     get weight 0, and tail rows of the last page are zeroed in LDS so that
//     whatever the cache holds there never reaches O.
#include <utility>

#include "mla_decode_common.h"

namespace mla {

using namespace dev;

// LDS of one decode workgroup besides the two page buffers: the softmax
// weights P of the current page in the output MFMA's operand order, and one
// float per row for the row sums the output waves need.
struct DecodeShared {
  char p[kPBytes];
  float x[2][kRowsPerBlock];    // per-row values of the two key halves (maxima, sums)
};

// One worker's pages for latent head g and row block rb: every segment in the
// worker's range [meta[0], meta[1]) .. [meta[2], meta[3]).
//
// Roles of the eight waves.  Scores and softmax: wave w takes query rows
// 16*(w%4) ..+15 (its Q, 16 x 576 bf16, sits in VGPRs) against keys
// 32*(w/4) ..+31 of each page; a row's maximum (first page) and sum combine
// the two halves through LDS.  Outputs: wave w owns output columns
// 64w ..+63 for all 64 rows (O^T, 64 x 64 fp32, in 16 MFMA accumulators),
// reading P of all rows from LDS and V columns 64w ..+63 only.
//
// kSingleHead: h_kv == 1, so a page's rows are contiguous 1152-byte rows and
// every stride is a compile-time constant.
//
// A segment whose scores rose too far above their reference (see the
// softmax below) is run a second time by the same workgroup, with each row's
// maximum over the segment as its reference.
template <bool kSingleHead>
__device__ __forceinline__ void decode_worker(const DecodeParams& p, char (*lds_page)[kPageBytes],
                                              DecodeShared& sh, const int32_t* meta, int g, int rb) {
  const uint32_t lds_base = (uint32_t)(uintptr_t)&lds_page[0][0];   // LDS byte address
  const uint32_t lds_p = (uint32_t)(uintptr_t)&sh.p[0];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp4 = lane >> 4;     // which 4-key / 8-wide k slice of an MFMA fragment
  const int col = lane & 15;      // row (or output column) within an MFMA tile
  const int rt = wave & 3;        // score row tile of this wave
  const int kh = wave >> 2;       // key half (32 keys of each page) of this wave's scores

  const int meta_b0 = ld_uniform(meta + 0), meta_b1 = ld_uniform(meta + 2);
  if (meta_b1 < meta_b0) return;                       // worker without pages
  // Compute cursor (cb, cpage, cend) and load cursor (lb, lpage, lend).
  int cb = meta_b0, cpage = ld_uniform(meta + 1), cend = segment_end(meta, p.seqlens, cb);
  if (cpage >= cend) return;
  int lb = cb, lpage = cpage, lend = cend, lp0 = cpage;
  const int nrb = p.row_blocks;
  bool lvalid = true;

  const int row_stride_bytes = kSingleHead ? kRowBytes : p.h_kv * kRowBytes;   // bytes between tokens
  const size_t page_stride_bytes = (size_t)kPage * row_stride_bytes;
  const uint32_t page_span = (uint32_t)(kPage * row_stride_bytes);              // resource size
  const char* kv_head = (const char*)p.kv + (size_t)g * kRowBytes;
  const uint32_t lane_src_off = (lane >> 3) * row_stride_bytes + ((lane & 7) ^ (lane >> 3)) * 16;

  // Page-independent per-lane LDS offsets; a fragment read adds the page
  // buffer's base and a compile-time offset below 64 KB.
  //   K: row col (+16 per key tile), 16-byte chunk 4*par + grp4 (+8 per 2 k-steps).
  //   V: row lane/4 (+16 per read), columns 64*wave + 16*d + 4*(lane%4).
  //   P: row 16*rt + col (write) or col (read, +16 per row tile), chunk grp4 (+4 per k-step).
  uint32_t kb_off[2], vb_off[4];
#pragma unroll
  for (int par = 0; par < 2; ++par) kb_off[par] = lds_tile_offset(col, 4 * par + grp4);
#pragma unroll
  for (int d = 0; d < 4; ++d)
    vb_off[d] = wave * 1024 + lds_tile_offset(lane >> 2, 2 * d + ((lane & 3) >> 1)) + 8 * (lane & 1);
  const uint32_t pw = lds_p + (16 * rt + col) * kPRowBytes + grp4 * 16;
  const uint32_t pr = lds_p + col * kPRowBytes + grp4 * 16;

  // Query row r of the block: its token and head.
  auto row_tok = [&](int r) __attribute__((always_inline)) {
    const int qrow = rb * kRowsPerBlock + r;
    return qrow < p.rows ? qrow / p.group : 0;
  };
  auto row_head = [&](int r) __attribute__((always_inline)) {
    const int qrow = rb * kRowsPerBlock + r;
    return qrow < p.rows ? g * p.group + (qrow - (qrow / p.group) * p.group) : 0;
  };
  const int srow = 16 * rt + col;      // this lane's score row

  // Q fragments of the score row for sequence b: lane (col, grp4) holds dims
  // 32*ks + 8*grp4 .. +7.
  bf16x8 qf[kDqk / 32];
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const bool ok = rb * kRowsPerBlock + srow < p.rows;
    const uint16_t* qp = p.q + ((size_t)(b * p.s_q + row_tok(srow)) * p.h_q + row_head(srow)) * kDqk + grp4 * 8;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
      u32x4 v = ok ? *(const u32x4*)(qp + ks * 32) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  };
  // First page in flight before anything else; the id of the page after it
  // is read now, one page ahead of its DMAs.
  int next_pid = 0;
  {
    const int page_id = ld_uniform(p.block_table + (size_t)lb * p.max_pages + page_in_order(lpage, lp0, lend, rb, nrb));
    lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
    stage_page<kLdsDmaPerWave>(kv_head + (size_t)page_id * page_stride_bytes, page_span, lane_src_off, row_stride_bytes,
               lds_base, wave);
    if (lvalid) next_pid = ld_uniform(p.block_table + (size_t)lb * p.max_pages + page_in_order(lpage, lp0, lend, rb, nrb));
  }

  int it = 0;
  while (true) {
    // ---------------- segment: pages [cpage, cend) of sequence cb ----------------
    const int b = cb;
    const int L = ld_uniform(p.seqlens + b);
    const int s0 = ld_uniform(p.num_splits + b);
    const int nsplit = ld_uniform(p.num_splits + b + 1) - s0;
    const int slot = s0 + (b == meta_b0 ? ld_uniform(meta + 4) : 0);
    const int seg_page0 = cpage;
    load_q(b);
    // Q is waited for here, once per segment, so that no wait inside the page
    // loop is left to count Q's loads (it would wait for the page DMAs too).
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    const int n_vis = p.causal ? L - p.s_q + row_tok(srow) + 1 : L;   // keys the score row may see
    // Fewest keys any row of the block sees (causal rows: the block's first token).
    const int n_vis_min = p.causal ? L - p.s_q + row_tok(0) + 1 : L;
    float m_ref = kNegInf;      // the score row's reference point (log2 units)
    bool second_pass = false;   // rerun with m_ref = the row's maximum over the segment
    float m_seen, l_run;        // largest score this lane has seen; its share of sum_j 2^(s_j - m_ref)
    int overflow;               // a score rose more than kOverflowThreshold above the reference
    f32x4 acc[4][4];

    while (true) {
      // ---------------- one pass over the segment's pages ----------------
      m_seen = kNegInf;
      l_run = 0.f;
      overflow = 0;
      // Output tiles, zeroed from an MFMA so that they are born in the
      // accumulation registers.
      {
        const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        const f32x4 zero4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zero8, zero8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[d][t] = zero4;
      }

      // The loop leaves at its bottom, so the tiles' loop-carried value has
      // the next page's first MFMA as its only use and every MFMA can
      // accumulate in place.
      while (true) {
        // Page `it` has landed in every wave's share, the buffer of page it-1
        // and the P buffer are free.
        wait_dma_all();
        __syncthreads();
        char* buf = lds_page[it & 1];
        const int ppage = page_in_order(cpage, seg_page0, cend, rb, nrb);   // the page this step processes
        const int valid = min(kPage, L - ppage * kPage);
        if (valid < kPage) {
          zero_tail_rows<kThreads>(buf, valid, tid);
          __syncthreads();
        }
        // The next page's DMAs go out one by one inside this page's MFMA
        // streams (below); its id was read a page ago.
        const bool dma = lvalid;
        const __amdgpu_buffer_rsrc_t dma_rsrc = page_resource(kv_head + (size_t)next_pid * page_stride_bytes, page_span);
        const uint32_t dma_dst = lds_base + ((it + 1) & 1) * kPageBytes;

        const uint32_t page_base = (uint32_t)(uintptr_t)buf;
        uint32_t kb[2], vb[4];
#pragma unroll
        for (int par = 0; par < 2; ++par) kb[par] = page_base + kb_off[par];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) vb[m4] = page_base + vb_off[m4];
        const int key0 = ppage * kPage;

        auto read_k = [&](int kt, int ks) __attribute__((always_inline)) {
          return *(lds_bf16x8*)(kb[ks & 1] + (uint32_t)((2 * kt * 9 + (ks >> 1)) * 1024));
        };
        // A operand of O^T += V^T P^T for output tile d of k-step kk: lane
        // (n = col, grp4) gets V[key][64*wave + 16d + n] for keys 32kk +
        // 4*grp4 + m and 32kk + 16 + 4*grp4 + m, from two transposing reads of
        // 4 rows x 16 columns (lane l fetches row l/4, columns 4*(l%4)..+3).
        auto read_v = [&](int kk, int d) __attribute__((always_inline)) {
          const uint32_t o0 = (uint32_t)((4 * kk + 0) * 9 * 1024);
          const uint32_t o1 = (uint32_t)((4 * kk + 2) * 9 * 1024);
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb[d] + o0));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb[d] + o1));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // B operand for output row tile t of k-step kk: lane (col, grp4) gets
        // P[16t + col][slots 8*grp4 .. +7 of k-step kk].
        auto read_p = [&](int kk, int t) __attribute__((always_inline)) {
          return *(lds_bf16x8*)(pr + (uint32_t)(t * 16 * kPRowBytes + kk * 64));
        };

        // ---- scores: S^T = K Q^T for key tiles 2kh, 2kh+1 (16 keys each) ----
        // 36 MFMAs, K fragments kKAhead reads ahead;
        // one DMA of the next page after MFMA kDmaStart + d * kDmaEvery of the
        // page (scores and outputs).
        constexpr int kKs = kDqk / 32;             // 18
        constexpr int kQk = 2 * kKs;               // 36 score MFMAs: 2 key tiles x 18 k-steps
        constexpr int kPv = 2 * 4 * 4;             // 32 output MFMAs: 2 k-steps x 4 column tiles x 4 row tiles
        constexpr int kKAhead = 8;
        constexpr int kDmaStart = 0;               // DMA d follows MFMA kDmaStart + d * kDmaEvery
        constexpr int kDmaEvery = 4;
        static_assert(kDmaStart + kDmaEvery * (kLdsDmaPerWave - 1) < kQk + kPv, "every DMA inside the streams");
        f32x4 s[2];
        bf16x8 kf[kQk];
        // Score MFMA G covers key tile 2*kh + G % 2 at k-step G / 2: the two
        // tiles' accumulation chains alternate.
#pragma unroll
        for (int r = 0; r < kKAhead; ++r) kf[r] = read_k(2 * kh + r % 2, r / 2);
        __builtin_amdgcn_sched_barrier(0);
        auto dma_step = [&]<int G>() __attribute__((always_inline)) {
          if constexpr (G >= kDmaStart && (G - kDmaStart) % kDmaEvery == 0 && (G - kDmaStart) / kDmaEvery < kLdsDmaPerWave) {
            if (dma) stage_tile<kLdsDmaPerWave>(dma_rsrc, lane_src_off, row_stride_bytes, dma_dst, wave, (G - kDmaStart) / kDmaEvery);
          }
        };
        auto qk_step = [&]<int G>() __attribute__((always_inline)) {
          constexpr int i = G % 2, ks = G / 2;
          const f32x4 c = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[i];
          s[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[G], qf[ks], c, 0, 0, 0);
          if constexpr (G + kKAhead < kQk) kf[G + kKAhead] = read_k(2 * kh + (G + kKAhead) % 2, (G + kKAhead) / 2);
          dma_step.template operator()<G>();
          __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... G>(std::integer_sequence<int, G...>) __attribute__((always_inline)) {
          (qk_step.template operator()<G>(), ...);
        }(std::make_integer_sequence<int, kQk>{});

        // The load cursor moves on and the id of the page after the next is
        // read here, where waiting for the scalar load costs nothing.
        if (lvalid) {
          lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
          if (lvalid) next_pid = ld_uniform(p.block_table + (size_t)lb * p.max_pages + page_in_order(lpage, lp0, lend, rb, nrb));
        }

        // ---- softmax weights (base 2) against the row reference ----
        // Lane (col, grp4) holds, for the score row, key key0 + 16*(2kh+i) +
        // 4*grp4 + e in s[i][e].  Keys the row may not see get weight 0;
        // masking is needed only on a page that holds such keys (the
        // sequence's last page, or causal rows), a uniform test.
        float x[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[i][e] = s[i][e];
        if (key0 + kPage > n_vis_min) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = key0 + 16 * (2 * kh + i) + 4 * grp4 + e;
              x[i][e] = key < n_vis ? x[i][e] : kNegInf;
            }
        }
        // This lane's maximum raw score (the scale is > 0), in log2 units.
        float xm = max2(max2(max2(x[0][0], x[0][1]), max2(x[0][2], x[0][3])),
                        max2(max2(x[1][0], x[1][1]), max2(x[1][2], x[1][3])));
        xm *= p.scale_log2;
        if (!second_pass && cpage == seg_page0) {
          // First page of the segment: the reference is the row's maximum over
          // the page (both key halves, swapped through LDS), so a sequence
          // that fits in one page has its largest weight exactly 1.
          const float hmax = row_max4(xm);
          if (grp4 == 0) sh.x[kh][srow] = hmax;
          __syncthreads();
          m_ref = max2(sh.x[0][srow], sh.x[1][srow]);
        }
        // A row with no reference yet that sees a key here, or a score far
        // above the reference, voids the segment's result for this pass.
        overflow |= xm > m_ref + kOverflowThreshold;
        m_seen = max2(m_seen, xm);
        const float mu = m_ref == kNegInf ? 0.f : m_ref;
        uint32_t pk[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float w0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i][2 * h], p.scale_log2, -mu));
            const float w1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i][2 * h + 1], p.scale_log2, -mu));
            l_run += w0 + w1;
            pk[i][h] = pack_bf16x2(w0, w1);
          }
        // Slot 8*grp4 + 4*i + e of k-step kk = kh holds key 32kh + 16i + 4*grp4 + e.
        *(__attribute__((address_space(3))) u32x4*)(pw + (uint32_t)(kh * 64)) =
            u32x4{pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
        __syncthreads();            // P of all 64 rows is in LDS

        // ---- outputs: O^T += V^T P^T, 4 column tiles x 4 row tiles per k-step ----
        // 32 MFMAs in issue order (kk, d, t); V fragments kVAhead ahead; the
        // four P fragments of a k-step read before its first MFMA.
        constexpr int kVAhead = 3;
        bf16x8 vf[2][4], pfr[2][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) pfr[0][t] = read_p(0, t);
#pragma unroll
        for (int d = 0; d < kVAhead; ++d) vf[0][d] = read_v(0, d);
        __builtin_amdgcn_sched_barrier(0);
        auto pv_step = [&]<int G>() __attribute__((always_inline)) {
          constexpr int n = G - kQk, kk = n / 16, d = (n % 16) / 4, t = n % 4;
          acc[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kk][d], pfr[kk][t], acc[d][t], 0, 0, 0);
          if constexpr (t == 3) {
            constexpr int nv = kk * 4 + d + kVAhead;   // next V fragment to read
            if constexpr (nv < 8) vf[nv / 4][nv % 4] = read_v(nv / 4, nv % 4);
          }
          if constexpr (kk == 0 && d == 1) pfr[1][t] = read_p(1, t);
          dma_step.template operator()<G>();
          __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... G>(std::integer_sequence<int, G...>) __attribute__((always_inline)) {
          (pv_step.template operator()<G + kQk>(), ...);
        }(std::make_integer_sequence<int, kPv>{});

        ++it;
        if (cpage + 1 == cend) break;
        ++cpage;
      }

      // Every wave is past its last output MFMA (sh.x below is free, and so is
      // the buffer of the segment's last page).  A second pass cannot
      // overflow (no score exceeds its row's maximum); it ends the loop anyway.
      if (!__syncthreads_or(overflow) || second_pass) break;
      // Some row of the block overflowed: the pass is void.  Run the segment
      // again with every row's maximum over it as the reference, so that no
      // weight exceeds 1.  The DMAs in flight (the worker's next page) are
      // drained and the load pipeline restarts at the segment's first page.
      {
        const float hmax = row_max4(m_seen);
        if (grp4 == 0) sh.x[kh][srow] = hmax;
        __syncthreads();
        m_ref = max2(sh.x[0][srow], sh.x[1][srow]);
      }
      second_pass = true;
      wait_dma_all();
      __syncthreads();
      lb = b;
      lpage = seg_page0;
      lend = cend;
      lp0 = seg_page0;
      cpage = seg_page0;
      {
        const int page_id = ld_uniform(p.block_table + (size_t)lb * p.max_pages + page_in_order(lpage, lp0, lend, rb, nrb));
        lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
        stage_page<kLdsDmaPerWave>(kv_head + (size_t)page_id * page_stride_bytes, page_span, lane_src_off, row_stride_bytes,
                   lds_base + (it & 1) * kPageBytes, wave);
        if (lvalid) next_pid = ld_uniform(p.block_table + (size_t)lb * p.max_pages + page_in_order(lpage, lp0, lend, rb, nrb));
      }
    }

    // ---------------- segment epilogue ----------------
    {
      // Row sums: each key half's share, swapped through LDS.
      const float l_half = row_sum4(l_run);
      if (grp4 == 0) sh.x[kh][srow] = l_half;
      __syncthreads();
      if (kh == 0 && grp4 == 0) {
        const float l_row = sh.x[0][srow] + sh.x[1][srow];
        const int qrow = rb * kRowsPerBlock + srow;
        const float lse_nat = l_row == 0.f ? kNegInf : (m_ref + __log2f(l_row)) * 0.69314718055994531f;
        if (qrow < p.rows) {
          if (nsplit == 1)
            p.lse[((size_t)b * p.h_q + row_head(srow)) * p.s_q + row_tok(srow)] = lse_nat;
          else
            p.ws_lse[(size_t)(slot * p.h_kv + g) * p.rows + qrow] = lse_nat;
        }
      }
      // O: lane (col, grp4) holds O[16t + col][64*wave + 16d + 4*grp4 + i] in acc[d][t][i].
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + col;
        const int qrow = rb * kRowsPerBlock + r;
        const float l = sh.x[0][r] + sh.x[1][r];
        const float inv = l == 0.f ? 0.f : 1.f / l;
        if (qrow < p.rows) {
          if (nsplit == 1) {
            uint16_t* op = p.o + ((size_t)(b * p.s_q + row_tok(r)) * p.h_q + row_head(r)) * kDv + 64 * wave + 4 * grp4;
#pragma unroll
            for (int d = 0; d < 4; ++d)
              *(u32x2*)(op + 16 * d) = u32x2{pack_bf16x2(acc[d][t][0] * inv, acc[d][t][1] * inv),
                                             pack_bf16x2(acc[d][t][2] * inv, acc[d][t][3] * inv)};
          } else {
            float* wp = p.ws_o + ((size_t)(slot * p.h_kv + g) * p.rows + qrow) * kDv + 64 * wave + 4 * grp4;
#pragma unroll
            for (int d = 0; d < 4; ++d) *(f32x4*)(wp + 16 * d) = acc[d][t] * inv;
          }
        }
      }
    }
    // The next segment's first page barrier orders these sh.x reads before
    // that segment rewrites it.

    // Next segment: the sequence after this one in the worker's range.
    if (cb == meta_b1) break;
    int nb = cb, np = cpage, ne = cend, n0 = seg_page0;
    if (!next_page(meta, p.seqlens, nb, np, ne, n0)) break;
    cb = nb;
    cpage = np;
    cend = ne;
  }
}

template <bool kSingleHead>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_page[2][kPageBytes];
  __shared__ __attribute__((aligned(16))) DecodeShared sh;
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
  decode_worker<kSingleHead>(p, lds_page, sh, p.meta + (size_t)worker * kMetaInts, g, rb);
}

template __global__ void mla_decode_kernel<true>(DecodeParams p);
template __global__ void mla_decode_kernel<false>(DecodeParams p);

}  // namespace mla
