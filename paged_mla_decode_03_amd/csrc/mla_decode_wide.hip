// Split-KV paged MLA decode kernel for gfx950 (MI355X), wide workgroups.
//
// What it computes is the same as mla_decode.hip: the MLA output equation of
// the deepseek.csdn.net FlashMLA article (section 2.2) after matrix
// absorption -- each absorbed query row (576 wide) attends over the
// sequence's cached latent rows [c^KV; k^R] and sums their first 512 columns
// with the softmax weights -- over one split of the paged cache (section
// 4.2(1): 64-token pages found through block_table, a split-KV kernel, then a
// combine kernel).
//
// This kernel serves heads with more than 128 query rows (several query
// tokens per sequence with 128 query heads) in workgroups of 128 rows, so
// that a page is staged into LDS once for twice as many rows as in the 64-row
// kernel.  There the matrix cores bound the work, and a CU's LDS-DMA ingest
// (about 64 KB in flight) is shared by half as many workgroups per page.  For
// heads of up to 128 rows the 64-row kernel is faster: its eight waves read
// LDS at twice the rate of these four, and it splits sequences half as often
// (fewer partials to write and combine).
//
// Work decomposition:
//   * One workgroup = 4 waves, one per SIMD, 512 registers each.  Wave w
//     takes query rows 32w ..+31 for the scores and output columns
//     128w ..+127 (all 128 rows) for O.
//   * Scores: S^T = K Q^T in 16x16 tiles: 4 key tiles x 2 row tiles x 18
//     k-steps of v_mfma_f32_16x16x32_bf16 (144 MFMAs per page).  The wave's
//     Q (32 x 576 bf16, 144 VGPRs) stays in registers for the segment; each K
//     fragment read from LDS feeds the two row tiles.  Eight accumulation
//     chains, so no MFMA waits for its predecessor.
//   * Softmax: a wave holds all 64 keys of its rows, so row maxima and sums
//     need only lane permutes, no LDS round trip.  P (bf16) goes to LDS.
//   * Outputs: O^T += V^T P^T, 8 column tiles x 8 row tiles x 2 k-steps (128
//     MFMAs per page) into 64 accumulators (256 registers) that only MFMAs
//     touch.  V^T comes from the transposing ds_read_b64_tr_b16.
//   * Pages move HBM -> LDS with buffer_load_dwordx4 ... lds, double
//     buffered; each wave issues 18 of a page's 72 DMAs among the previous
//     page's score MFMAs.
//   * LDS: two 72 KB page buffers and 16 KB of P fill the 160 KB.  P rows
//     are 128 bytes with their 16-byte units XOR-swizzled by row pair, so
//     neither its writes nor its reads conflict across 16 consecutive rows.
//   * Softmax in base 2 against a per-row reference point: the row's maximum
//     over the segment's first page.  The overflow rule with its in-place
//     second pass, the key masking and the page order are those of
//     mla_decode.hip.
#include <utility>

#include "mla_decode_common.h"

namespace mla {

using namespace dev;

namespace {

// Score MFMAs with their accumulators in VGPRs.  A kernel with 512 registers
// per wave gets every builtin MFMA in its AGPR form, and the AGPRs are all
// taken by the output tiles (256 registers), so the 32 score accumulators are
// placed here by hand.  The hazard checker does not see these MFMAs: their
// sources are LDS/global loads (no VALU write shortly before), each chain's
// accumulator is touched only by these MFMAs, and the score stream ends with
// qk_drain(), which waits out the last result before anything reads the
// scores.
__device__ inline f32x4 mfma_qk_first(bf16x8 a, bf16x8 b) {
  f32x4 d;
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ inline void mfma_qk(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// 24 wait states: more than an 8-pass XDL write needs before a VALU, LDS or
// memory instruction reads or overwrites its result.  It names all eight
// score tiles as operands, so no read of any of them can be placed before it.
__device__ inline void qk_drain(f32x4 (&s)[4][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]),
                 "+v"(s[2][0]), "+v"(s[2][1]), "+v"(s[3][0]), "+v"(s[3][1]));
}

// Byte offset of 16-byte unit u (0..7) of row r of the P buffer.
__device__ inline uint32_t p_unit_offset(int r, int u) {
  return (uint32_t)(r * kWidePRowBytes + ((u ^ ((r >> 1) & 7)) * 16));
}

}  // namespace

// One worker's pages for latent head g and row block rb (128 query rows):
// every segment in the worker's range [meta[0], meta[1]) .. [meta[2], meta[3]).
template <bool kSingleHead>
__device__ __forceinline__ void wide_worker(const DecodeParams& p, char (*lds_page)[kPageBytes], char* lds_w,
                                            const int32_t* meta, int g, int rb) {
  const uint32_t lds_base = (uint32_t)(uintptr_t)&lds_page[0][0];   // LDS byte address
  const uint32_t lds_p = (uint32_t)(uintptr_t)lds_w;
  float* sx = (float*)lds_w;      // row sums for the epilogue (P is free then) ...
  int* flags = (int*)(lds_w + kWideRows * 4);   // ... and one overflow flag per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp4 = lane >> 4;     // which 4-key / 8-wide k slice of an MFMA fragment
  const int col = lane & 15;      // row (or output column) within an MFMA tile

  const int meta_b0 = ld_uniform(meta + 0), meta_b1 = ld_uniform(meta + 2);
  if (meta_b1 < meta_b0) return;                       // worker without pages
  // Compute cursor (cb, cpage, cend) and load cursor (lb, lpage, lend).
  int cb = meta_b0, cpage = ld_uniform(meta + 1), cend = segment_end(meta, p.seqlens, cb);
  if (cpage >= cend) return;
  int lb = cb, lpage = cpage, lend = cend, lp0 = cpage;
  size_t lrow = 0;   // lb * max_pages: the load cursor's block_table row
  const int nrb = p.row_blocks;
  bool lvalid = true;

  const int row_stride_bytes = kSingleHead ? kRowBytes : p.h_kv * kRowBytes;   // bytes between tokens
  const size_t page_stride_bytes = (size_t)kPage * row_stride_bytes;
  const uint32_t page_span = (uint32_t)(kPage * row_stride_bytes);              // resource size
  const char* kv_head = (const char*)p.kv + (size_t)g * kRowBytes;
  const uint32_t lane_src_off = (lane >> 3) * row_stride_bytes + ((lane & 7) ^ (lane >> 3)) * 16;
  const WaveTiles<kWideDmaPerWave> tiles(wave, row_stride_bytes);
  const uint32_t wave_tiles_lds = (uint32_t)(wave * kWideDmaPerWave * 1024);   // the wave's first tile in a page buffer

  // Page-independent per-lane LDS offsets; a fragment read adds the page
  // buffer's base and a compile-time offset below 64 KB.
  //   K: row col (+16 per key tile), 16-byte chunk 4*par + grp4 (+8 per 2 k-steps).
  //   V: row lane/4 (+16 per read), columns 128*wave + 16*d + 4*(lane%4); the
  //      offsets of column tiles d and d+4 differ by one LDS tile (1 KB).
  //   P: row col (+16 per row tile), unit 4*kk + grp4.
  // One register per operand: with the XOR swizzle, chunk 4 + c differs
  // from chunk c by bit 6 of the byte offset, chunk 2d + c (c < 2) from c by
  // bits 5-6 (d << 5), and P unit 4 + u from u by bit 6; the page and P
  // buffers are 1 KB aligned and the added row and tile offsets are
  // multiples of 1 KB or 2 KB, so the XOR applies to the full address.
  const uint32_t kb_off = lds_tile_offset(col, grp4);
  const uint32_t vb_off = lds_tile_offset(lane >> 2, 16 * wave + ((lane & 3) >> 1)) + 8 * (lane & 1);
  const uint32_t pr_off0 = lds_p + p_unit_offset(col, grp4);
  auto pr_off = [&](int kk) __attribute__((always_inline)) { return pr_off0 ^ (uint32_t)(64 * kk); };
  // Score rows of this wave: 32*wave + 16*j + col (the swizzle of a P row
  // depends on col only, so the write offset is the read offset plus whole rows).
  const uint32_t pw_base = (uint32_t)(2 * wave) * 16 * kWidePRowBytes;

  // Query row r of the block: its token and head.
  auto row_tok = [&](int r) __attribute__((always_inline)) {
    const int qrow = rb * kWideRows + r;
    return qrow < p.rows ? qrow / p.group : 0;
  };
  auto row_head = [&](int r) __attribute__((always_inline)) {
    const int qrow = rb * kWideRows + r;
    return qrow < p.rows ? g * p.group + (qrow - (qrow / p.group) * p.group) : 0;
  };
  int srow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) srow[j] = 32 * wave + 16 * j + col;

  // Q fragments of the two score rows for sequence b: lane (col, grp4) holds
  // dims 32*ks + 8*grp4 .. +7.
  bf16x8 qf[2][kDqk / 32];
  auto load_q = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = rb * kWideRows + srow[j] < p.rows;
      const uint16_t* qp =
          p.q + ((size_t)(b * p.s_q + row_tok(srow[j])) * p.h_q + row_head(srow[j])) * kDqk + grp4 * 8;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        u32x4 v = ok ? *(const u32x4*)(qp + ks * 32) : u32x4{0, 0, 0, 0};
        qf[j][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  // First page in flight before anything else; the id of the page after it
  // is read now, one page ahead of its DMAs.
  int next_pid = 0;
  {
    const int first_pid = page_id(p, lb, page_in_order(lpage, lp0, lend, rb, nrb));
    lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
    stage_page<kWideDmaPerWave>(page_rsrc(kv_head, first_pid, p.num_pages, page_stride_bytes, page_span),
                                lane_src_off, lds_base + wave_tiles_lds, tiles);
    lrow = (size_t)lb * p.max_pages;
    if (lvalid) next_pid = page_id(p, lb, page_in_order(lpage, lp0, lend, rb, nrb));
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
    int n_vis[2];                // keys each score row may see
#pragma unroll
    for (int j = 0; j < 2; ++j) n_vis[j] = p.causal ? L - p.s_q + row_tok(srow[j]) + 1 : L;
    // Fewest keys any row of the block sees (causal rows: the block's first token).
    const int n_vis_min = p.causal ? L - p.s_q + row_tok(0) + 1 : L;
    float m_ref[2] = {kNegInf, kNegInf};   // the score rows' reference points (log2 units)
    bool second_pass = false;   // rerun with m_ref = the row's maximum over the segment
    float m_seen[2], l_run[2];  // largest score this lane has seen; its share of sum_j 2^(s_j - m_ref)
    float l_bf[2];              // its share of the same sum over the bf16-rounded weights (O's normaliser)
    float l_row[2];             // the rows' sums sum_j 2^(s_j - m_ref) at the end of a pass
    int overflow;               // a score rose more than kOverflowThreshold above the reference
    f32x4 acc[8][8];

    while (true) {
      // ---------------- one pass over the segment's pages ----------------
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        m_seen[j] = kNegInf;
        l_run[j] = 0.f;
        l_bf[j] = 0.f;
      }
      overflow = 0;
      {
        const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        const f32x4 zero4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zero8, zero8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[d][t] = zero4;
      }

      while (true) {
        // Page `it` has landed in every wave's share, the buffer of page it-1
        // and the P buffer are free.
        wait_dma_all();
        __syncthreads();
        char* buf = lds_page[it & 1];
        // The page this step processes, needed only where its keys can reach
        // n_vis_min (rows past the sequence end to zero, keys to mask): the
        // page order moves a page by at most nrb - 1 places, so before page
        // n_vis_min / 64 - nrb + 1 of the segment's walk every key is
        // visible.
        const bool attn = cpage > n_vis_min / kPage - nrb;
        int ppage = 0;
        if (attn) {
          ppage = page_in_order(cpage, seg_page0, cend, rb, nrb);
          const int valid = min(kPage, L - ppage * kPage);
          if (valid < kPage) {
            zero_tail_rows<kWideThreads>(buf, valid, tid);
            __syncthreads();
          }
        }
        // The next page's DMAs go out in every step, so that the score stream
        // holds no branch: with no page left they read from a resource of
        // size 0 and write zeros into the free buffer.
        const __amdgpu_buffer_rsrc_t dma_rsrc =
            page_rsrc(kv_head, lvalid ? next_pid : -1, p.num_pages, page_stride_bytes, page_span);
        const uint32_t dma_m0 = lds_base + ((it + 1) & 1) * kPageBytes + wave_tiles_lds;

        const uint32_t page_base = (uint32_t)(uintptr_t)buf;
        const uint32_t kb0 = page_base + kb_off, vb0 = page_base + vb_off;
        const uint32_t kb[2] = {kb0, kb0 ^ 64u};
        const int key0 = ppage * kPage;

        auto read_k = [&](int kt, int ks) __attribute__((always_inline)) {
          return *(lds_bf16x8*)(kb[ks & 1] + (uint32_t)((2 * kt * 9 + (ks >> 1)) * 1024));
        };
        // A operand of O^T += V^T P^T for output tile d of k-step kk: lane
        // (n = col, grp4) gets V[key][128*wave + 16d + n] for keys 32kk +
        // 4*grp4 + m and 32kk + 16 + 4*grp4 + m, from two transposing reads of
        // 4 rows x 16 columns (lane l fetches row l/4, columns 4*(l%4)..+3).
        auto read_v = [&](int kk, int d) __attribute__((always_inline)) {
          const uint32_t a = (vb0 ^ (uint32_t)((d & 3) << 5)) + (uint32_t)((d >> 2) * 1024);
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + (uint32_t)((4 * kk + 0) * 9 * 1024)));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + (uint32_t)((4 * kk + 2) * 9 * 1024)));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // B operand for output row tile t of k-step kk: lane (col, grp4) gets
        // P[16t + col][slots 8*grp4 .. +7 of k-step kk].
        auto read_p = [&](int kk, int t) __attribute__((always_inline)) {
          return *(lds_bf16x8*)(pr_off(kk) + (uint32_t)(t * 16 * kWidePRowBytes));
        };

        // ---- scores: S^T = K Q^T, 4 key tiles x 2 row tiles ----
        // K fragment F = 4*ks + kt feeds MFMAs 2F and 2F+1 (row tiles 0 and
        // 1); fragments are read kKAhead ahead.  The page's 272 MFMAs (144
        // score, 128 output) are numbered in issue order, and DMA d of the
        // next page follows MFMA kDmaStart + kDmaEvery * d.  The DMAs stay in
        // the score stream: issued among the output MFMAs they keep their
        // resource and predicate live there, and the registers run out.
        constexpr int kKs = kDqk / 32;             // 18
        constexpr int kFrags = 4 * kKs;            // 72 K fragments per page
        constexpr int kQk = 2 * kFrags;            // 144 score MFMAs
        constexpr int kPv = 128;                   // 128 output MFMAs
        constexpr int kKAhead = 10;
        constexpr int kDmaStart = 0;
        constexpr int kDmaEvery = 8;
        static_assert(kDmaStart + kDmaEvery * (kWideDmaPerWave - 1) < kQk, "every DMA inside the score stream");
        auto dma_step = [&]<int G>() __attribute__((always_inline)) {
          if constexpr (G >= kDmaStart && (G - kDmaStart) % kDmaEvery == 0 && (G - kDmaStart) / kDmaEvery < kWideDmaPerWave) {
            stage_tile<kWideDmaPerWave, (G - kDmaStart) / kDmaEvery>(dma_rsrc, lane_src_off, dma_m0, tiles);
          }
        };
        f32x4 s[4][2];
        bf16x8 kf[kFrags];
#pragma unroll
        for (int r = 0; r < kKAhead; ++r) kf[r] = read_k(r % 4, r / 4);
        __builtin_amdgcn_sched_barrier(0);
        auto qk_step = [&]<int F>() __attribute__((always_inline)) {
          constexpr int kt = F % 4, ks = F / 4;
          if constexpr (ks == 0)
            s[kt][0] = mfma_qk_first(kf[F], qf[0][ks]);
          else
            mfma_qk(s[kt][0], kf[F], qf[0][ks]);
          dma_step.template operator()<2 * F>();
          if constexpr (ks == 0)
            s[kt][1] = mfma_qk_first(kf[F], qf[1][ks]);
          else
            mfma_qk(s[kt][1], kf[F], qf[1][ks]);
          if constexpr (F == kFrags - 1) qk_drain(s);
          if constexpr (F + kKAhead < kFrags) kf[F + kKAhead] = read_k((F + kKAhead) % 4, (F + kKAhead) / 4);
          dma_step.template operator()<2 * F + 1>();
          __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... F>(std::integer_sequence<int, F...>) __attribute__((always_inline)) {
          (qk_step.template operator()<F>(), ...);
        }(std::make_integer_sequence<int, kFrags>{});

        // The load cursor moves on and the id of the page after the next is
        // read; its scalar load lands during the softmax.  Inside a segment
        // that is a few scalar instructions (for two row blocks the page
        // order is a select, the table row's offset is kept, and the table
        // index is clamped into the row instead of branching around the
        // load); a segment's end takes the full walk to the next sequence.
        if (lvalid) {
          if (lpage + 1 < lend) {
            ++lpage;
            int j;
            if (nrb == 2) {
              const int jj = lpage - lp0 - 1;
              const int base = lp0 + 1 + (jj & ~1);
              j = (jj < 0 || base + 2 > lend) ? lpage : base + ((jj & 1) ^ rb);
            } else {
              j = page_in_order(lpage, lp0, lend, rb, nrb);
            }
            const int pid = ld_uniform(p.block_table + lrow + min(j, p.max_pages - 1));
            next_pid = j < p.max_pages ? pid : -1;
          } else {
            lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
            lrow = (size_t)lb * p.max_pages;
            if (lvalid) next_pid = page_id(p, lb, page_in_order(lpage, lp0, lend, rb, nrb));
          }
        }

        // ---- softmax weights (base 2) against the row references ----
        // Lane (col, grp4) holds, for score row srow[j], key key0 + 16*kt +
        // 4*grp4 + e in s[kt][j][e].  Keys a row may not see get weight 0;
        // masking is needed only on a page that holds such keys (the
        // sequence's last page, or causal rows), a uniform test.
        const bool first_page = !second_pass && cpage == seg_page0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float x[4][4];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[kt][e] = s[kt][j][e];
          if (attn && key0 + kPage > n_vis_min) {
            // Key key0 + 16*kt + 4*grp4 + e is visible iff 16*kt + e < lim:
            // one subtraction per row, compile-time offsets per key (the key
            // indices themselves would be formed on every page).
            const int lim = n_vis[j] - key0 - 4 * grp4;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int e = 0; e < 4; ++e) x[kt][e] = 16 * kt + e < lim ? x[kt][e] : kNegInf;
          }
          // This lane's maximum raw score (the scale is > 0), in log2 units.
          float xm = kNegInf;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) xm = max2(xm, max2(max2(x[kt][0], x[kt][1]), max2(x[kt][2], x[kt][3])));
          xm *= p.scale_log2;
          // First page of the segment: the reference is the row's maximum
          // over the page, so a sequence that fits in one page has its
          // largest weight exactly 1.
          if (first_page) m_ref[j] = row_max4(xm);
          // A row with no reference yet that sees a key here, or a score far
          // above the reference, voids the segment's result for this pass.
          overflow |= xm > m_ref[j] + kOverflowThreshold;
          m_seen[j] = max2(m_seen[j], xm);
          const float mu = m_ref[j] == kNegInf ? 0.f : m_ref[j];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            uint32_t pk[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float w0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * kk + i][2 * h], p.scale_log2, -mu));
                const float w1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * kk + i][2 * h + 1], p.scale_log2, -mu));
                l_run[j] += w0 + w1;
                pk[i][h] = pack_bf16x2(w0, w1);
                l_bf[j] = add_bf16x2(l_bf[j], pk[i][h]);
              }
            // Slot 8*grp4 + 4*i + e of k-step kk holds key 32kk + 16i + 4*grp4 + e.
            *(__attribute__((address_space(3))) u32x4*)(pr_off(kk) + pw_base + (uint32_t)(j * 16 * kWidePRowBytes)) =
                u32x4{pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
          }
        }
        __syncthreads();            // P of all 128 rows is in LDS

        // ---- outputs: O^T += V^T P^T, 8 column tiles x 8 row tiles per k-step ----
        // 128 MFMAs in issue order (kk, d, t); V fragments kVAhead column
        // tiles ahead; the P fragments of k-step 1 are read during column
        // tile 6 of k-step 0.
        constexpr int kVAhead = 4;
        bf16x8 vf[2][8], pfr[2][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) pfr[0][t] = read_p(0, t);
#pragma unroll
        for (int d = 0; d < kVAhead; ++d) vf[0][d] = read_v(0, d);
        __builtin_amdgcn_sched_barrier(0);
        auto pv_step = [&]<int n>() __attribute__((always_inline)) {
          constexpr int kk = n / 64, d = (n % 64) / 8, t = n % 8;
          acc[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kk][d], pfr[kk][t], acc[d][t], 0, 0, 0);
          if constexpr (t == 7) {
            constexpr int nv = kk * 8 + d + kVAhead;   // next V fragment to read
            if constexpr (nv < 16) vf[nv / 8][nv % 8] = read_v(nv / 8, nv % 8);
          }
          if constexpr (kk == 0 && d == 6) pfr[1][t] = read_p(1, t);
          dma_step.template operator()<kQk + n>();
          __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... n>(std::integer_sequence<int, n...>) __attribute__((always_inline)) {
          (pv_step.template operator()<n>(), ...);
        }(std::make_integer_sequence<int, kPv>{});

        ++it;
        if (cpage + 1 == cend) break;
        ++cpage;
      }

      // End of the pass.  Once every wave is past its last output MFMA the P
      // buffer is free: each wave leaves its rows' sums there for the
      // epilogue and a flag for whether any of its rows overflowed.  (A
      // second pass cannot overflow -- no score exceeds its row's maximum --
      // and ends the loop anyway.)
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        l_row[j] = row_sum4(l_run[j]);
        const float l_norm = row_sum4(l_bf[j]);
        if (grp4 == 0) sx[srow[j]] = l_norm;
      }
      const bool wave_overflow = __builtin_amdgcn_ballot_w64(overflow != 0) != 0;
      if (lane == 0) flags[wave] = wave_overflow;
      __syncthreads();
      if (!(flags[0] | flags[1] | flags[2] | flags[3]) || second_pass) break;
      // Some row of the block overflowed: the pass is void.  Run the segment
      // again with every row's maximum over it as the reference, so that no
      // weight exceeds 1.  The DMAs in flight (the worker's next page) are
      // drained and the load pipeline restarts at the segment's first page.
#pragma unroll
      for (int j = 0; j < 2; ++j) m_ref[j] = row_max4(m_seen[j]);
      second_pass = true;
      wait_dma_all();
      __syncthreads();
      lb = b;
      lpage = seg_page0;
      lend = cend;
      lp0 = seg_page0;
      cpage = seg_page0;
      {
        const int first_pid = page_id(p, lb, page_in_order(lpage, lp0, lend, rb, nrb));
        lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
        stage_page<kWideDmaPerWave>(page_rsrc(kv_head, first_pid, p.num_pages, page_stride_bytes, page_span),
                                    lane_src_off, lds_base + (it & 1) * kPageBytes + wave_tiles_lds, tiles);
        lrow = (size_t)lb * p.max_pages;
        if (lvalid) next_pid = page_id(p, lb, page_in_order(lpage, lp0, lend, rb, nrb));
      }
    }

    // ---------------- segment epilogue ----------------
    // The row sums are in sx (written at the end of the pass).
    {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (grp4 == 0) {
          const int qrow = rb * kWideRows + srow[j];
          const float lse_nat = l_row[j] == 0.f ? kNegInf : (m_ref[j] + __log2f(l_row[j])) * 0.69314718055994531f;
          if (qrow < p.rows) {
            if (nsplit == 1)
              p.lse[((size_t)b * p.h_q + row_head(srow[j])) * p.s_q + row_tok(srow[j])] = lse_nat;
            else
              p.ws_lse[(size_t)(slot * p.h_kv + g) * p.rows + qrow] = lse_nat;
          }
        }
      }
      // O: lane (col, grp4) holds O[16t + col][128*wave + 16d + 4*grp4 + i] in acc[d][t][i].
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = 16 * t + col;
        const int qrow = rb * kWideRows + r;
        const float l = sx[r];
        const float inv = l == 0.f ? 0.f : 1.f / l;
        if (qrow < p.rows) {
          if (nsplit == 1) {
            uint16_t* op = p.o + ((size_t)(b * p.s_q + row_tok(r)) * p.h_q + row_head(r)) * kDv + 128 * wave + 4 * grp4;
#pragma unroll
            for (int d = 0; d < 8; ++d)
              *(u32x2*)(op + 16 * d) = u32x2{pack_bf16x2(acc[d][t][0] * inv, acc[d][t][1] * inv),
                                             pack_bf16x2(acc[d][t][2] * inv, acc[d][t][3] * inv)};
          } else {
            float* wp = p.ws_o + ((size_t)(slot * p.h_kv + g) * p.rows + qrow) * kDv + 128 * wave + 4 * grp4;
#pragma unroll
            for (int d = 0; d < 8; ++d) *(f32x4*)(wp + 16 * d) = acc[d][t] * inv;
          }
        }
      }
    }
    // The next segment's first page barrier orders these sx reads before that
    // segment writes P over them.

    // Next segment: the sequence after this one in the worker's range.
    if (cb == meta_b1) break;
    int nb = cb, np = cpage, ne = cend, n0 = seg_page0;
    if (!next_page(meta, p.seqlens, nb, np, ne, n0)) break;
    cb = nb;
    cpage = np;
    cend = ne;
  }
  // The last page step issued DMAs (of zeros) into the free buffer: they
  // land before the workgroup gives its LDS back.
  wait_dma_all();
}

template <bool kSingleHead>
__global__ __launch_bounds__(kWideThreads, 1) void mla_decode_wide_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_page[2][kPageBytes];
  __shared__ __attribute__((aligned(1024))) char lds_w[kWidePBytes];
  // Block -> (worker, latent head, row block), XCD-aware as in the 64-row
  // kernel: the row blocks of one (worker, head) get ids on the same XCD,
  // issued back to back.
  const int xcd = blockIdx.x % kNumXcd;
  const int k = blockIdx.x / kNumXcd;
  const int rb = k % p.row_blocks;
  const int grp = (k / p.row_blocks) * kNumXcd + xcd;
  if (grp >= p.num_workers * p.h_kv) return;
  const int worker = grp / p.h_kv;
  const int g = grp - worker * p.h_kv;
  wide_worker<kSingleHead>(p, lds_page, lds_w, p.meta + (size_t)worker * kMetaInts, g, rb);
}

template __global__ void mla_decode_wide_kernel<true>(DecodeParams p);
template __global__ void mla_decode_wide_kernel<false>(DecodeParams p);

}  // namespace mla
