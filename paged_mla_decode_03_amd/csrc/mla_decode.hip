// Split-KV paged MLA decode kernel for gfx950 (MI355X), 64 query rows per
// workgroup.
//
// What it computes: the MLA output equation of the deepseek.csdn.net FlashMLA
// article (section 2.2) after matrix absorption -- each absorbed query row
// (576 wide) attends over the sequence's cached latent rows [c^KV; k^R] and
// sums their first 512 columns (c^KV) with the softmax weights -- over one
// split of the paged cache (section 4.2(1): 64-token pages found through
// block_table, a split-KV forward kernel, then a combine kernel).
//
// Work decomposition (8 waves, two per SIMD; heads of up to 128 query rows --
// larger heads use mla_decode_wide.hip):
//   * One workgroup = 64 query rows of one latent head over the page range
//     the scheduler gave its worker.  The workgroups that serve the other row
//     block of the same head read the same pages; they are dispatched back to
//     back on the same XCD, and take the pages in a rotated order, so the
//     second read hits L2.
//   * Score waves 0..3: wave s holds Q of rows 16s..16s+15 (72 VGPRs) and, per
//     half page of 32 keys, computes S^T = K Q^T (2 key tiles x 18 k-steps of
//     v_mfma_f32_16x16x32_bf16, K fragments from LDS), the softmax (a wave
//     holds all 32 keys of its rows: row maxima and sums by lane permutes)
//     and writes its rows of P (bf16) to LDS.
//   * Output waves 4..7: wave 4+o owns output columns 128o..128o+127 for all
//     64 rows (32 accumulator tiles that only MFMAs touch) and accumulates
//     O^T += V^T P^T for one half page per step (8 column tiles x 4 row
//     tiles; V^T through the transposing ds_read_b64_tr_b16).
//   * Step k of a segment: the score waves work on half page k+1 while the
//     output waves work on half page k, so on each SIMD one wave's softmax and
//     LDS waits overlap the other's MFMAs.  One workgroup barrier per step.
//   * LDS: a ring of four 36 KB half-page slots (half page q in slot q % 4,
//     as 36 tiles of 1 KB, 8 rows x 8 chunks of 16 bytes with the chunks
//     XOR-swizzled by row) and two 4 KB P buffers (half page q's weights in
//     buffer q % 2).  Pages move HBM -> LDS with buffer_load_dwordx4 ... lds
//     (no VGPR staging; the buffer resource bounds every read to the page).
//     During step k the output waves issue the DMAs of half page k+3 (9
//     each, before their MFMAs) and, before the step's barrier, wait for
//     their share of half page k+2, which the score waves read in step k+1.
//     (bf16; the fp8 cache's staging below uses all eight waves.)
//   * Softmax runs in base 2 with the scale folded into one multiply.  Each
//     row keeps a reference point m (its maximum over the segment's first half
//     page) and accumulates unnormalised weights 2^(s - m) <= 2^48; that is
//     exact math, and bf16/fp32 have the range for it (sums stay below 2^65
//     times the largest cached value for 2^17 keys).  The output tiles are
//     therefore never rescaled.  Should a later score exceed a row's
//     reference by more than 48, the pass is void and the workgroup runs the
//     segment again with each row's maximum over the segment as its
//     reference, where no weight exceeds 1.  For attention scores of any
//     ordinary spread the second pass never runs.
//   * Keys a query may not see (tail slots of the last page, causal future)
//     get weight 0, and rows past the sequence end are zeroed in LDS so that
//     whatever the cache holds there never reaches O.
#include <utility>

#include "mla_decode_common.h"

namespace mla {

using namespace dev;

namespace {

constexpr int kHalfRows = 32;                         // keys per half page
constexpr int kHalfBytes = kHalfRows * kRowBytes;     // 36864 bytes per ring slot
constexpr int kRingSlots = 4;
constexpr int kRawHalfBytes = kHalfRows * kDqk;       // a half page of fp8 codes: 18432 bytes
constexpr int kRawUnits = kRawHalfBytes / 1024;       // 18 wave-wide 1 KB DMAs
constexpr int kPRowBytes = 2 * kHalfRows;           // one row of P: 32 bf16
constexpr int kPBytes = kRowsPerBlock * kPRowBytes;   // 4 KB per P buffer
// A half page is 36 wave-wide DMAs: tile row r (rows 8r..8r+7) x 9 tile
// columns.  Output wave 4+r issues tile row r, before its MFMAs.  The score
// waves, whose scores and softmax make the longer half of a step, issue
// none and keep no load cursor of their own in the step loop (a DMA stalls
// its wave at issue for about a hundred cycles while the memory queue is
// full, and the output waves otherwise wait at the step's barrier).
constexpr int kScoreDma = 0;
constexpr int kOutputDma = 9;
static_assert(kScoreDma + kOutputDma == kHalfRows * kChunksPerRow / 64 / 4, "9 tile columns per tile row");

// page_in_order for at most two row blocks, all this kernel meets (it
// serves heads of up to 128 query rows in 64-row workgroups): no division.
__device__ inline int page_in_order_le2(int page, int p0, int end, int rb, int nrb) {
  const int j = page - p0 - 1;
  if (j < 0 || nrb == 1) return page;
  const int base = p0 + 1 + (j & ~1);
  return base + 2 > end ? page : base + ((j & 1) ^ rb);
}

// Byte offset of 16-byte unit u (0..3) of row r of a P buffer: rows of 64
// bytes, units XOR-swizzled by r / 4, so 16 consecutive rows read or write
// 16 distinct 16-byte bank groups.
__device__ inline uint32_t p_unit_offset(int r, int u) {
  return (uint32_t)(r * kPRowBytes + ((u ^ ((r >> 2) & 3)) * 16));
}

// Wait until at most n of this wave's vector memory operations (its own
// DMAs of one half page) are in flight, in inline assembly like wait_dma_all.
template <int n>
__device__ inline void wait_dma_keep() {
  static_assert(n >= 0 && n <= 9, "wait counts written out below");
  if constexpr (n == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  if constexpr (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  if constexpr (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  if constexpr (n == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  if constexpr (n == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  if constexpr (n == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  if constexpr (n == 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  if constexpr (n == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  if constexpr (n == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
}

}  // namespace

// bf16 cache: a ring of four half-page slots.  fp8 cache: three bf16 slots
// (each half page is converted into one a step before its first reader,
// into the slot its predecessor's predecessor has left) and two slots of raw
// fp8 codes that the DMAs fill a step ahead of the conversion.  Both fill
// the same 155,920 bytes.
template <bool kFp8>
struct DecodeShared {
  char ring[kRingSlots][kHalfBytes];
  char p[2][kPBytes];
  float l[kRowsPerBlock];           // row sums at the end of a segment
  int flags[4];                     // overflow votes of the score waves
};
template <>
struct DecodeShared<true> {
  char ring[kRingSlots - 1][kHalfBytes];
  char raw[2][kRawHalfBytes];
  char p[2][kPBytes];
  float l[kRowsPerBlock];
  int flags[4];
};
static_assert(sizeof(DecodeShared<true>) == sizeof(DecodeShared<false>), "same LDS for both caches");

// One role's loop over the worker's segments.  Both roles run the same
// sequence of steps and barriers; each is compiled on its own so that the
// score waves' Q and the output waves' accumulators never share registers.
//
// kFp8: the cache holds fp8 codes (OCP E4M3, one fp32 scale for the cache).
// A half page then moves HBM -> registers (each lane loads 8-byte chunks of
// 8 codes, the same chunks every time: 5 per lane in the score waves, 4 in
// the output waves, 2304 per half page) one step before it is needed, and in
// the next step it is converted, exactly, to bf16 and written into its ring
// slot in the same swizzled layout the DMAs fill, so the scores, softmax and
// outputs are unchanged.  The cache's scale is folded into the score scale
// and the output normaliser (p.scale_log2 and p.out_scale).
template <bool kSingleHead, bool scorer, bool kFp8>
__device__ __forceinline__ void decode_role(const DecodeParams& p, DecodeShared<kFp8>& sh, const int32_t* meta, int g,
                                            int rb) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp4 = lane >> 4;
  const int col = lane & 15;

  const int meta_b0 = ld_uniform(meta + 0), meta_b1 = ld_uniform(meta + 2);
  if (meta_b1 < meta_b0) return;
  int cb = meta_b0, cpage = ld_uniform(meta + 1), cend = segment_end(meta, p.seqlens, cb);
  if (cpage >= cend) return;
  const int nrb = p.row_blocks;

  constexpr int kElemBytes = kFp8 ? 1 : 2;              // bytes per cached value
  constexpr int kRowBytesIn = kDqk * kElemBytes;          // one latent row of one head in the cache
  const int row_stride_bytes = kSingleHead ? kRowBytesIn : p.h_kv * kRowBytesIn;
  const size_t page_stride_bytes = (size_t)kPage * row_stride_bytes;
  const uint32_t page_span = (uint32_t)(kPage * row_stride_bytes);
  const char* kv_head = (const char*)p.kv + (size_t)g * kRowBytesIn;
  const uint32_t lane_src_off = (lane >> 3) * row_stride_bytes + ((lane & 7) ^ (lane >> 3)) * 16;
  const uint32_t ring_base = (uint32_t)(uintptr_t)&sh.ring[0][0];
  // Ring slot of global half page i (i >= 0).
  auto ring_slot = [](int i) __attribute__((always_inline)) { return kFp8 ? i % (kRingSlots - 1) : i & (kRingSlots - 1); };
  const uint32_t p_base = (uint32_t)(uintptr_t)&sh.p[0][0];

  // Load cursor over half pages (each wave keeps its own copy and issues its
  // share of the DMAs): page (lb, lpage) of segment [lp0, lend), half lhalf;
  // gq counts half pages issued.
  int lb = cb, lpage = cpage, lend = cend, lp0 = cpage, lhalf = 0, gq = 0;
  bool lvalid = true;
  int lpid = page_id(p, lb, page_in_order_le2(lpage, lp0, lend, rb, nrb));
  const int ow = wave - 4;   // output wave index
  constexpr int kDma = scorer ? kScoreDma : kOutputDma;   // this wave's DMAs per half page
  constexpr int kCol0 = scorer ? kOutputDma : 0;          // its first tile column
  const int trow = wave & 3;                              // its tile row of a half page
  // Issue this wave's DMAs of the load cursor's half page into its ring slot
  // and advance the cursor; returns whether anything was issued.
  auto issue_half = [&]() __attribute__((always_inline)) {
    if (!lvalid) return false;
    const __amdgpu_buffer_rsrc_t rsrc = page_rsrc(kv_head, lpid, p.num_pages, page_stride_bytes, page_span);
    const uint32_t dst =
        ring_base + (uint32_t)(ring_slot(gq) * kHalfBytes) + (uint32_t)((trow * 9 + kCol0) * 1024);
    const uint32_t soff0 = (uint32_t)((kHalfRows * lhalf + 8 * trow) * row_stride_bytes + kCol0 * 128);
    [&]<int... j>(std::integer_sequence<int, j...>) __attribute__((always_inline)) {
      (lds_dma16_at<j * 1024, j * 128>(dst, lane_src_off, rsrc, soff0), ...);
    }(std::make_integer_sequence<int, kDma>{});
    ++gq;
    if (lhalf == 0) {
      lhalf = 1;
    } else {
      lhalf = 0;
      lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
      if (lvalid) lpid = page_id(p, lb, page_in_order_le2(lpage, lp0, lend, rb, nrb));
    }
    return true;
  };
  // End of a step: wait for this wave's share of the half page the score
  // waves read next (all but the DMAs just issued, if any).
  auto wait_next = [&](bool issued) __attribute__((always_inline)) {
    if constexpr (kFp8) return;   // plain loads: the compiler waits for them where they are used
    if (issued)
      wait_dma_keep<kDma>();
    else
      wait_dma_all();
  };

  // fp8 staging.  A half page of codes is 18 wave-wide DMAs of 1 KB, unit u
  // = bytes 1024u .. +1023 of its 32 x 576 codes in row order, landing at the
  // same offset of a raw slot; this wave issues units s, s + 8 (and s + 16)
  // for s = (wave + 4) % 8 (the output waves 4 and 5 take the last two), and
  // in the next step each lane converts the 16 codes its own DMAs brought --
  // so only the wave's own DMAs are waited for, and no barrier -- exactly to
  // bf16 and writes them into the half page's ring slot in the swizzled
  // layout the bf16 DMAs fill.
  constexpr int kUnits = scorer ? 2 : 3;
  const int unit0 = (wave + 4) & 7;
  const int units = unit0 + 16 < kRawUnits ? 3 : 2;       // 3 for waves 4 and 5
  uint32_t raw_base = 0;
  uint32_t raw_voff[kUnits], raw_t0[kUnits], raw_t1[kUnits];
  if constexpr (kFp8) {
    raw_base = (uint32_t)(uintptr_t)&sh.raw[0][0];
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int b = 1024 * (unit0 + 8 * i) + 16 * lane;    // code index in the half page
      const int r = b / kDqk, c = b - (b / kDqk) * kDqk;   // row and first column (a multiple of 16)
      raw_voff[i] = (uint32_t)(r * row_stride_bytes + c);
      raw_t0[i] = (uint32_t)lds_tile_offset(r, c / 8);
      raw_t1[i] = (uint32_t)lds_tile_offset(r, c / 8 + 1);
    }
  }
  int f8_idx = -1;   // global half-page index whose codes wait in a raw slot (-1: none)
  auto load_half = [&]() __attribute__((always_inline)) {
    if (!lvalid) return false;
    const __amdgpu_buffer_rsrc_t rsrc = page_rsrc(kv_head, lpid, p.num_pages, page_stride_bytes, page_span);
    const uint32_t soff = (uint32_t)(kHalfRows * lhalf * row_stride_bytes);
    const uint32_t dst = raw_base + (uint32_t)((gq & 1) * kRawHalfBytes) + (uint32_t)(unit0 * 1024);
#pragma unroll
    for (int i = 0; i < kUnits; ++i)
      if (i < 2 || units == 3) lds_dma16(dst + (uint32_t)(i * 8 * 1024), raw_voff[i], rsrc, soff);
    f8_idx = gq;
    ++gq;
    if (lhalf == 0) {
      lhalf = 1;
    } else {
      lhalf = 0;
      lvalid = next_page(meta, p.seqlens, lb, lpage, lend, lp0);
      if (lvalid) lpid = page_id(p, lb, page_in_order_le2(lpage, lp0, lend, rb, nrb));
    }
    return true;
  };
  // Codes of half page f8_idx -> bf16 (exact: every E4M3 value is a bf16
  // value) into its ring slot, after this wave's own DMAs of it have landed.
  auto convert_half = [&]() __attribute__((always_inline)) {
    wait_dma_all();
    const uint32_t raw = raw_base + (uint32_t)((f8_idx & 1) * kRawHalfBytes) + (uint32_t)(unit0 * 1024 + 16 * lane);
    char* half = &sh.ring[ring_slot(f8_idx)][0];
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      if (i < 2 || units == 3) {
        const u32x4 codes = *(const __attribute__((address_space(3))) u32x4*)(raw + (uint32_t)(i * 8 * 1024));
        u32x4 o[2];
        // Two codes to two bf16 in one instruction (scale 1: every E4M3
        // value is a bf16 value, so the conversion is exact).
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[h], 1.0f, false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[h], 1.0f, true);
          o[h >> 1][2 * (h & 1)] = __builtin_bit_cast(uint32_t, lo);
          o[h >> 1][2 * (h & 1) + 1] = __builtin_bit_cast(uint32_t, hi);
        }
        *(u32x4*)(half + raw_t0[i]) = o[0];
        *(u32x4*)(half + raw_t1[i]) = o[1];
      }
    }
    f8_idx = -1;
  };
  // One step's staging: bf16 issues its DMAs of half page gbase+k+3; fp8
  // converts half page gbase+k+2 (loaded in the previous step) and loads
  // half page gbase+k+3.  Returns whether DMAs were issued.
  auto stage_step = [&](int target) __attribute__((always_inline)) {
    if constexpr (kFp8) {
      if (f8_idx == target - 1) convert_half();
      if (gq == target) load_half();
      return false;
    } else {
      return gq == target && issue_half();
    }
  };

  // Score waves: per-lane offsets.  K: row col (+16 per key tile), 16-byte
  // chunk 4*par + grp4 (+8 per 2 k-steps).  P write: rows 16*wave + col.
  const int srow = 16 * (wave & 3) + col;
  uint32_t kb_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) kb_off[par] = lds_tile_offset(col, 4 * par + grp4);
  const uint32_t pw_off = p_unit_offset(srow, grp4);
  // Output waves: V columns 128*ow + 16*d + 4*(lane%4), rows lane/4 (+16);
  // P rows 16*t + col, unit grp4.
  uint32_t vb_off[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    vb_off[d] = lds_tile_offset(lane >> 2, 16 * (ow & 3) + 2 * d + ((lane & 3) >> 1)) + 8 * (lane & 1);
  const uint32_t pr_off = p_unit_offset(col, grp4);   // + 16 rows per row tile (the swizzle repeats every 16 rows)

  auto row_tok = [&](int r) __attribute__((always_inline)) {
    const int qrow = rb * kRowsPerBlock + r;
    return qrow < p.rows ? qrow / p.group : 0;
  };
  auto row_head = [&](int r) __attribute__((always_inline)) {
    const int qrow = rb * kRowsPerBlock + r;
    return qrow < p.rows ? g * p.group + (qrow - (qrow / p.group) * p.group) : 0;
  };

  // Prologue of the worker: half pages 0 and 1 in flight, wait for 0 (fp8:
  // half page 0 converted, half page 1 in registers).
  if constexpr (kFp8) {
    load_half();
    convert_half();
    load_half();
  } else {
    issue_half();
    const bool issued = issue_half();
    wait_next(issued);
  }

  int gbase = 0;   // global half-page index of the segment's first half page
  while (true) {
    // ---------------- segment: pages [cpage, cend) of sequence cb ----------------
    const int b = cb;
    const int L = ld_uniform(p.seqlens + b);
    const int s0 = ld_uniform(p.num_splits + b);
    const int nsplit = ld_uniform(p.num_splits + b + 1) - s0;
    const int slot = s0 + (b == meta_b0 ? ld_uniform(meta + 4) : 0);
    const int seg_page0 = cpage;
    const int nhalf = 2 * (cend - cpage);
    // Score waves: Q of the score row, the row's visible keys.
    bf16x8 qf[kDqk / 32];
    int n_vis = 0;
    if constexpr (scorer) {
      const bool ok = rb * kRowsPerBlock + srow < p.rows;
      const uint16_t* qp = p.q + ((size_t)(b * p.s_q + row_tok(srow)) * p.h_q + row_head(srow)) * kDqk + grp4 * 8;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        u32x4 v = ok ? *(const u32x4*)(qp + ks * 32) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // score waves issue no DMAs
      n_vis = p.causal ? L - p.s_q + row_tok(srow) + 1 : L;
    }
    const int n_vis_min = p.causal ? L - p.s_q + row_tok(0) + 1 : L;
    // Half pages that can hold keys at or past n_vis_min (rows to zero past
    // the sequence end, keys to mask) start at step index hp_attn: the page
    // order moves a page by at most one place, so the half page at step hp
    // lies in page seg_page0 + hp/2 + 1 or below, whose keys end before
    // n_vis_min while hp < hp_attn.  Earlier steps skip the page-order
    // arithmetic.
    const int hp_attn = 2 * (n_vis_min / kPage - seg_page0 - 1);
    float m_ref = kNegInf;
    // Derived from m_ref wherever it is set: the exponent offset (0 for a row
    // without a reference) and the score above which the pass overflows.
    float m_mu = 0.f, m_lim = kNegInf;
    bool second_pass = false;
    float m_seen, l_run, l_bf;   // l_run: exact sum of the weights (for lse); l_bf: of their bf16 roundings (for O)
    int overflow;
    f32x4 acc[8][4];

    while (true) {
      // ---------------- one pass over the segment's half pages ----------------
      m_seen = kNegInf;
      l_run = 0.f;
      l_bf = 0.f;
      overflow = 0;
      if constexpr (!scorer) {
        const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        const f32x4 zero4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zero8, zero8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[d][t] = zero4;
      }
      // Every half page of this pass has landed before a score wave reads it
      // (the previous step's wait and barrier); rows past the sequence end
      // are zeroed here, at the top of the step before their first reader.
      __syncthreads();

      // Step k = -1 .. nhalf-1: score waves on half page k+1, output waves on k.
      for (int k = -1; k < nhalf; ++k) {
        // Tail of half page k+1 (read by the score waves now and the output
        // waves next step): rows past the sequence end hold anything.
        // Page of half page k+1 (its tail here, its masking below).
        const bool attn = k + 1 >= hp_attn;
        int ppage1 = 0;
        if (attn && k + 1 < nhalf) {
          const int hp = k + 1;
          ppage1 = page_in_order_le2(seg_page0 + hp / 2, seg_page0, cend, rb, nrb);
          const int valid = min(kHalfRows, L - ppage1 * kPage - kHalfRows * (hp & 1));
          if (valid < kHalfRows) {
            char* half = &sh.ring[ring_slot(gbase + hp)][0];
            for (int i = max(valid, 0) * kChunksPerRow + tid; i < kHalfRows * kChunksPerRow; i += kThreads) {
              const int r = i / kChunksPerRow;
              const int c = i - r * kChunksPerRow;
              *(u32x4*)(half + lds_tile_offset(r, c)) = u32x4{0, 0, 0, 0};
            }
            __syncthreads();
          }
        }
        if constexpr (scorer) {
          if (k + 1 < nhalf) {
            // ---- scores of half page hp = k+1: S^T = K Q^T, key tiles 0, 1 ----
            const int hp = k + 1;
            const int key0 = ppage1 * kPage + kHalfRows * (hp & 1);
            const uint32_t half_base = ring_base + (uint32_t)(ring_slot(gbase + hp) * kHalfBytes);
            uint32_t kb[2];
#pragma unroll
            for (int par = 0; par < 2; ++par) kb[par] = half_base + kb_off[par];
            auto read_k = [&](int kt, int ks) __attribute__((always_inline)) {
              return *(lds_bf16x8*)(kb[ks & 1] + (uint32_t)((2 * kt * 9 + (ks >> 1)) * 1024));
            };
            constexpr int kKs = kDqk / 32;
            constexpr int kQk = 2 * kKs;             // 36 MFMAs
            constexpr int kKAhead = 8;
            f32x4 s[2];
            bf16x8 kf[kQk];
#pragma unroll
            for (int r = 0; r < kKAhead; ++r) kf[r] = read_k(r % 2, r / 2);
            __builtin_amdgcn_sched_barrier(0);
            auto qk_step = [&]<int G>() __attribute__((always_inline)) {
              constexpr int i = G % 2, ks = G / 2;
              const f32x4 c = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[i];
              s[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[G], qf[ks], c, 0, 0, 0);
              if constexpr (G + kKAhead < kQk) kf[G + kKAhead] = read_k((G + kKAhead) % 2, (G + kKAhead) / 2);
              __builtin_amdgcn_sched_barrier(0);
            };
            [&]<int... G>(std::integer_sequence<int, G...>) __attribute__((always_inline)) {
              (qk_step.template operator()<G>(), ...);
            }(std::make_integer_sequence<int, kQk>{});

            // ---- softmax weights (base 2) of the 32 keys ----
            // Lane (col, grp4) holds key key0 + 16*i + 4*grp4 + e in s[i][e].
            float x[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int e = 0; e < 4; ++e) x[i][e] = s[i][e];
            if (attn && key0 + kHalfRows > n_vis_min) {
              // Key key0 + 16*i + 4*grp4 + e is visible iff 16*i + e < lim.
              const int lim = n_vis - key0 - 4 * grp4;
#pragma unroll
              for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) x[i][e] = 16 * i + e < lim ? x[i][e] : kNegInf;
            }
            float xm = max2(max2(max2(x[0][0], x[0][1]), max2(x[0][2], x[0][3])),
                            max2(max2(x[1][0], x[1][1]), max2(x[1][2], x[1][3])));
            xm *= p.scale_log2;
            // The segment's first half page sets each row's reference.
            if (!second_pass && hp == 0) {
              m_ref = row_max4(xm);
              m_mu = m_ref == kNegInf ? 0.f : m_ref;
              m_lim = m_ref + kOverflowThreshold;
            }
            overflow |= xm > m_lim;
            m_seen = max2(m_seen, xm);
            const float mu = m_mu;
            uint32_t pk[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float w0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i][2 * h], p.scale_log2, -mu));
                const float w1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i][2 * h + 1], p.scale_log2, -mu));
                l_run += w0 + w1;
                pk[i][h] = pack_bf16x2(w0, w1);
                l_bf = add_bf16x2(l_bf, pk[i][h]);
              }
            // Slot 8*grp4 + 4*i + e holds key 16i + 4*grp4 + e of the half page.
            *(__attribute__((address_space(3))) u32x4*)(p_base + (uint32_t)((hp & 1) * kPBytes) + pw_off) =
                u32x4{pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
          }
          // This wave's share of half page gbase+k+3, then wait for its share
          // of half page gbase+k+2 (see the output waves).
          if constexpr (kFp8 || kDma > 0) {
            const bool issued = stage_step(gbase + k + 3);
            wait_next(issued);
          }
        } else {
          // ---- output waves: DMAs of half page gbase+k+3, outputs of half page k ----
          // (The last step of the previous segment already issued this
          // segment's half page gbase+2: a step issues only when the load
          // cursor stands at gbase+k+3, so the ring slot it fills, that of
          // half page k-1, is free.)
          const bool issued = stage_step(gbase + k + 3);
          if (k >= 0) {
            const uint32_t half_base = ring_base + (uint32_t)(ring_slot(gbase + k) * kHalfBytes);
            uint32_t vb[4];
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) vb[m4] = half_base + vb_off[m4];
            const uint32_t pr = p_base + (uint32_t)((k & 1) * kPBytes) + pr_off;
            // A operand: lane (n = col, grp4) gets V[key][128*ow + 16d + n] for
            // keys 4*grp4 + m and 16 + 4*grp4 + m (two transposing reads).
            auto read_v = [&](int d) __attribute__((always_inline)) {
              const uint32_t a = vb[d & 3] + (uint32_t)((d >> 2) * 1024);
              const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
              const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + (uint32_t)(2 * 9 * 1024)));
              return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            auto read_p = [&](int t) __attribute__((always_inline)) {
              return *(lds_bf16x8*)(pr + (uint32_t)(t * 16 * kPRowBytes));
            };
            constexpr int kVAhead = 3;
            bf16x8 vf[8], pfr[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) pfr[t] = read_p(t);
#pragma unroll
            for (int d = 0; d < kVAhead; ++d) vf[d] = read_v(d);
            __builtin_amdgcn_sched_barrier(0);
            auto pv_step = [&]<int n>() __attribute__((always_inline)) {
              constexpr int d = n / 4, t = n % 4;
              acc[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d], pfr[t], acc[d][t], 0, 0, 0);
              if constexpr (t == 3 && d + kVAhead < 8) vf[d + kVAhead] = read_v(d + kVAhead);
              __builtin_amdgcn_sched_barrier(0);
            };
            [&]<int... n>(std::integer_sequence<int, n...>) __attribute__((always_inline)) {
              (pv_step.template operator()<n>(), ...);
            }(std::make_integer_sequence<int, 32>{});
          }
          // Half page gbase+k+2 (read by the score waves next step) has landed.
          wait_next(issued);
        }
        __syncthreads();
      }

      // End of the pass: the score waves leave their rows' sums and an
      // overflow vote in LDS.  (A second pass cannot overflow.)
      if constexpr (scorer) {
        const float l_row = row_sum4(l_run);
        const float l_norm = row_sum4(l_bf);
        if (grp4 == 0) sh.l[srow] = l_norm;
        const bool wave_overflow = __builtin_amdgcn_ballot_w64(overflow != 0) != 0;
        if (lane == 0) sh.flags[wave] = wave_overflow;
        if (grp4 == 0) {
          const int qrow = rb * kRowsPerBlock + srow;
          if (qrow < p.rows) {
            // lse of the pass; rewritten by a second pass if there is one.
            const float lse_nat = l_row == 0.f ? kNegInf : (m_ref + __log2f(l_row)) * 0.69314718055994531f;
            if (nsplit == 1)
              p.lse[((size_t)b * p.h_q + row_head(srow)) * p.s_q + row_tok(srow)] = lse_nat;
            else
              p.ws_lse[(size_t)(slot * p.h_kv + g) * p.rows + qrow] = lse_nat;
          }
        }
      }
      __syncthreads();
      if (!(sh.flags[0] | sh.flags[1] | sh.flags[2] | sh.flags[3]) || second_pass) break;
      // Overflow: rerun the segment with each row's maximum as reference.
      // The output waves drain their DMAs and restart the load pipeline at
      // the segment's first half page.
      if constexpr (scorer) {
        m_ref = row_max4(m_seen);
        m_mu = m_ref == kNegInf ? 0.f : m_ref;
        m_lim = m_ref + kOverflowThreshold;
      }
      second_pass = true;
      {
        wait_dma_all();
        lb = b;
        lpage = seg_page0;
        lend = cend;
        lp0 = seg_page0;
        lhalf = 0;
        lvalid = true;
        gq = gbase;
        lpid = page_id(p, lb, page_in_order_le2(lpage, lp0, lend, rb, nrb));
        if constexpr (kFp8) {
          f8_idx = -1;   // drop what was loaded ahead; the pass reloads from its start
          load_half();
          convert_half();
          load_half();
        } else {
          issue_half();
          const bool issued = issue_half();
          wait_next(issued);
        }
      }
    }

    // ---------------- segment epilogue (output waves) ----------------
    if constexpr (!scorer) {
      // O: lane (col, grp4) holds O[16t + col][128*ow + 16d + 4*grp4 + i] in acc[d][t][i].
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + col;
        const int qrow = rb * kRowsPerBlock + r;
        const float l = sh.l[r];
        const float inv = l == 0.f ? 0.f : p.out_scale / l;
        if (qrow < p.rows) {
          if (nsplit == 1) {
            uint16_t* op = p.o + ((size_t)(b * p.s_q + row_tok(r)) * p.h_q + row_head(r)) * kDv + 128 * ow + 4 * grp4;
#pragma unroll
            for (int d = 0; d < 8; ++d)
              *(u32x2*)(op + 16 * d) = u32x2{pack_bf16x2(acc[d][t][0] * inv, acc[d][t][1] * inv),
                                             pack_bf16x2(acc[d][t][2] * inv, acc[d][t][3] * inv)};
          } else {
            float* wp = p.ws_o + ((size_t)(slot * p.h_kv + g) * p.rows + qrow) * kDv + 128 * ow + 4 * grp4;
#pragma unroll
            for (int d = 0; d < 8; ++d) *(f32x4*)(wp + 16 * d) = acc[d][t] * inv;
          }
        }
      }
      // The stores count in vmcnt with the DMAs: let them finish, so that the
      // step waits of the next segment count only DMAs.
      wait_dma_all();
    }
    gbase += nhalf;

    // Next segment: the sequence after this one in the worker's range.  The
    // next step's barrier orders these sh.l reads before their next writes.
    if (cb == meta_b1) break;
    // (The steps index the segment's pages from seg_page0; the cursor steps
    // on from its last page.)
    int nb = cb, np = cend - 1, ne = cend, n0 = seg_page0;
    if (!next_page(meta, p.seqlens, nb, np, ne, n0)) break;
    cb = nb;
    cpage = np;
    cend = ne;
  }
  // Waves leave with no DMA in flight into this workgroup's LDS.
  wait_dma_all();
}

template <bool kSingleHead>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) DecodeShared<false> sh;
  const int xcd = blockIdx.x % kNumXcd;
  const int k = blockIdx.x / kNumXcd;
  const int rb = k % p.row_blocks;
  const int grp = (k / p.row_blocks) * kNumXcd + xcd;
  if (grp >= p.num_workers * p.h_kv) return;
  const int worker = grp / p.h_kv;
  const int g = grp - worker * p.h_kv;
  const int32_t* meta = p.meta + (size_t)worker * kMetaInts;
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
    decode_role<kSingleHead, true, false>(p, sh, meta, g, rb);
  else
    decode_role<kSingleHead, false, false>(p, sh, meta, g, rb);
}

// The same kernel over an fp8 cache (see decode_role's kFp8).
template <bool kSingleHead>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_fp8_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) DecodeShared<true> sh;
  const int xcd = blockIdx.x % kNumXcd;
  const int k = blockIdx.x / kNumXcd;
  const int rb = k % p.row_blocks;
  const int grp = (k / p.row_blocks) * kNumXcd + xcd;
  if (grp >= p.num_workers * p.h_kv) return;
  const int worker = grp / p.h_kv;
  const int g = grp - worker * p.h_kv;
  const int32_t* meta = p.meta + (size_t)worker * kMetaInts;
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
    decode_role<kSingleHead, true, true>(p, sh, meta, g, rb);
  else
    decode_role<kSingleHead, false, true>(p, sh, meta, g, rb);
}

template __global__ void mla_decode_kernel<true>(DecodeParams p);
template __global__ void mla_decode_kernel<false>(DecodeParams p);
template __global__ void mla_decode_fp8_kernel<true>(DecodeParams p);
template __global__ void mla_decode_fp8_kernel<false>(DecodeParams p);

}  // namespace mla
