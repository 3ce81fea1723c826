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
//   * One workgroup = 4 waves = 128 query rows of one latent head, over the
//     page range the scheduler gave its worker.  All 128 rows share each
//     staged page, so every latent row is read from HBM once per workgroup.
//   * Wave v owns query rows 32v..32v+31.  Its absorbed Q (32 x 576 bf16) sits
//     in VGPRs as MFMA B fragments for the whole segment; its output
//     O^T (512 x 32 fp32) sits in 16 MFMA 32x32 accumulators.
//   * Per page: S^T = K * Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from
//     LDS, B = Q), online softmax in the accumulator layout (each lane holds
//     one query row), then O^T += V^T * P^T with the same MFMA (A = V columns
//     from LDS, B = P straight from the S^T accumulators, no shuffle).
//   * Pages move HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging),
//     double-buffered: page i+1 is in flight while page i is computed.  16-byte
//     chunks are XOR-swizzled by row (chunk c of row r lives at slot
//     c ^ (r & 7)) so that the MFMA fragment reads hit distinct LDS banks.
//   * Softmax runs in base 2 with the scale folded into one multiply.  Each
//     row keeps a reference point m (its maximum over the segment's first
//     page) and accumulates unnormalised weights 2^(s - m) <= 2^16; that is
//     exact math, and bf16/fp32 have the range for it.  The output tile is
//     therefore never rescaled: only MFMAs touch it.  Should a later page
//     exceed a row's reference by more than 16, the workgroup restarts the
//     segment from its first page with the larger reference (each restart
//     raises a reference by more than 16, so restarts are few and finite;
//     for ordinary attention scores they never happen).
//   * Keys a query may not see (tail slots of the last page, causal future)
//     get weight 0, and tail rows of the last page are zeroed in LDS so that
//     whatever the cache holds there never reaches O.
#include "mla_kernels.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) const uint16_t lds_u16;

constexpr float kRestartThreshold = 16.0f;   // log2 units: weights stay <= 2^16
constexpr float kNegInf = -__builtin_huge_valf();

__device__ inline int pages_of(int seqlen) { return (seqlen + kPage - 1) / kPage; }

// LDS layout of a staged page: 72 tiles of 1 KB, tile (a, b) = rows 8a..8a+7 x
// 16-byte chunks 8b..8b+7 at byte (9a + b) * 1024; inside a tile, chunk c of
// row r sits at slot 8 * (r % 8) + ((c % 8) ^ (r % 8)).  The XOR spreads the
// 8 rows an MFMA fragment read touches over distinct banks, and one wave-wide
// 16-byte DMA fills exactly one tile.
__device__ inline int lds_tile_offset(int r, int c) {
  return ((r >> 3) * 9 + (c >> 3)) * 1024 + ((r & 7) * 8 + ((c & 7) ^ (r & 7))) * 16;
}

// Stage one page of latent head g into LDS with 72 wave-wide DMAs (18 per
// wave).  Lane u of the DMA for tile (a, b) fetches row 8a + u/8, chunk
// 8b + ((u%8) ^ (u/8)), so its source address is a wave-uniform base (SGPRs)
// plus one per-lane offset, and its destination is the tile's wave-uniform
// LDS address.  All 64 rows are fetched; rows past the sequence end are
// zeroed afterwards by zero_tail_rows().
__device__ inline void stage_page(const char* page_head, uint32_t lane_src_off, int row_stride_bytes,
                                  char* dst, int wave) {
#pragma unroll
  for (int k = 0; k < kLdsDmaPerWave; ++k) {
    const int j = k * kWaves + wave;            // tile index 9a + b, wave-uniform
    const int a = j / 9, b = j - (j / 9) * 9;
    const char* src = page_head + (a * 8 * row_stride_bytes + b * 128);
    __builtin_amdgcn_global_load_lds((const void*)(src + lane_src_off), (lds_void*)(dst + j * 1024), 16, 0, 0);
  }
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

__device__ inline float wave_max_pair(float x) {
  // rows live in lanes l and l^32; combine the two halves
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

struct Cursor {
  int b, page, end;   // current sequence, page index, end page of this segment
  bool valid;
};

__device__ inline void cursor_begin(Cursor& c, const int32_t* meta, const int32_t* seqlens) {
  c.b = meta[0];
  c.page = meta[1];
  c.end = meta[2] == meta[0] ? meta[3] : pages_of(seqlens[meta[0]]);
  c.valid = meta[2] >= meta[0] && c.page < c.end;
}

__device__ inline void cursor_next(Cursor& c, const int32_t* meta, const int32_t* seqlens) {
  if (++c.page < c.end) return;
  const int b_last = meta[2];
  for (int b = c.b + 1; b <= b_last; ++b) {
    const int end = b == b_last ? meta[3] : pages_of(seqlens[b]);
    if (end > 0) {
      c.b = b;
      c.page = 0;
      c.end = end;
      return;
    }
  }
  c.valid = false;
}

}  // namespace

// kSingleHead: h_kv == 1, so a page's rows are contiguous 1152-byte rows and
// every stride is a compile-time constant.
template <bool kSingleHead>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_page[2][kPageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int half = lane >> 5;     // which 8-wide k slice of an MFMA fragment this lane holds
  const int col = lane & 31;      // query row within the wave's tile / MFMA column

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

  const int32_t* meta = p.meta + (size_t)worker * kMetaInts;
  Cursor cur;
  cursor_begin(cur, meta, p.seqlens);
  if (!cur.valid) return;
  Cursor ld = cur;

  const int row_stride_bytes = kSingleHead ? kRowBytes : p.h_kv * kRowBytes;   // bytes between tokens
  const size_t page_stride_bytes = (size_t)kPage * row_stride_bytes;
  const char* kv_head = (const char*)p.kv + (size_t)g * kRowBytes;
  const uint32_t lane_src_off = (lane >> 3) * row_stride_bytes + ((lane & 7) ^ (lane >> 3)) * 16;
  auto page_ptr = [&](const Cursor& c) {
    const int page_id = __builtin_amdgcn_readfirstlane(p.block_table[(size_t)c.b * p.max_pages + c.page]);
    return kv_head + (size_t)page_id * page_stride_bytes;
  };

  // This lane's query row.
  const int qrow = rb * kRowsPerBlock + wave * kRowsPerWave + col;
  const bool row_ok = qrow < p.rows;
  const int q_tok = row_ok ? qrow / p.group : 0;
  const int q_head = g * p.group + (row_ok ? qrow - q_tok * p.group : 0);

  // First page in flight before anything else.
  stage_page(page_ptr(ld), lane_src_off, row_stride_bytes, lds_page[0], wave);
  cursor_next(ld, meta, p.seqlens);

  int it = 0;
  while (true) {
    // ---------------- segment: pages [cur.page, cur.end) of sequence cur.b ----------------
    const int b = cur.b;
    const int L = p.seqlens[b];
    const int s0 = p.num_splits[b];
    const int nsplit = p.num_splits[b + 1] - s0;
    const int slot = s0 + (b == meta[0] ? meta[4] : 0);
    const int n_vis_min = p.causal ? L - p.s_q + 1 : L;
    const int n_vis_row = p.causal ? L - p.s_q + q_tok + 1 : L;
    const Cursor seg_start = cur;

    bf16x8 qf[kDqk / 16];
    {
      const uint16_t* qp = p.q + ((size_t)(b * p.s_q + q_tok) * p.h_q + q_head) * kDqk + half * 8;
#pragma unroll
      for (int ks = 0; ks < kDqk / 16; ++ks) {
        u32x4 v = row_ok ? *(const u32x4*)(qp + ks * 16) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    float m_ref = kNegInf;      // this row's reference point (log2 units)
    float m_seen = kNegInf;     // largest score seen in the segment
    float l_run = 0.f;          // this lane's share of sum_j 2^(s_j - m_ref)
    int restart = 0;            // this lane's row outgrew its reference
    f32x16 acc[kDv / 32];

    // One attempt per reference point; the output tiles are zeroed here and
    // only MFMAs touch them until the segment epilogue.
    while (true) {
#pragma unroll
    for (int nt = 0; nt < kDv / 32; ++nt) acc[nt] = f32x16{};
    l_run = 0.f;
    bool done = false;          // the segment's last page has been computed
    int vote = 0;

    while (true) {
      // Page `it` has landed in every wave's share; the buffer of page it-1
      // is free; and every wave has voted on a restart.
      __builtin_amdgcn_s_waitcnt(0);
      vote = __syncthreads_or(restart);
      if (vote || done) break;
      char* buf = lds_page[it & 1];
      const int valid = min(kPage, L - cur.page * kPage);
      if (valid < kPage) {
        zero_tail_rows(buf, valid, tid);
        __syncthreads();
      }
      if (ld.valid) {
        stage_page(page_ptr(ld), lane_src_off, row_stride_bytes, lds_page[(it + 1) & 1], wave);
        cursor_next(ld, meta, p.seqlens);
      }

      // The page is processed as two halves of 32 keys (mt = 0, 1), each a
      // 32-key S^T tile, its weights, and its two 16-key k-steps of the output.
      const int key0 = cur.page * kPage;
      const bool need_mask = key0 + kPage > n_vis_min;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        // Per-lane bases of this half page's fragment reads (its rows start
        // 36 KB into the page); every read is one of them plus a compile-time
        // offset.  They are recomputed here from the lane id rather than kept
        // live across the loop, and the empty asm statements stop the compiler
        // from hoisting them again or turning base + offset into an OR that
        // the DS immediate offset cannot absorb.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int c32 = ln & 31, hf = ln >> 5;
        const uint32_t hp = (uint32_t)(uintptr_t)(buf + mt * 36 * 1024);
        uint32_t kb[4], vb[2][4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          kb[k4] = hp + lds_tile_offset(c32, 2 * k4 + hf);
          asm volatile("" : "+v"(kb[k4]));
        }
#pragma unroll
        for (int par = 0; par < 2; ++par) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vb[par][j] = hp + lds_tile_offset(4 * hf + j, 4 * par + (c32 >> 3)) + (c32 & 7) * 2;
            asm volatile("" : "+v"(vb[par][j]));
          }
        }

        // ---- S^T = K * Q^T over 36 k-steps of 16 ----
        // Lane (col, half) reads key 32*mt + col, chunk 2*ks + half, which sits
        // at kb[ks % 4] + (ks/4) KB.
        f32x16 s;
#pragma unroll
        for (int ks = 0; ks < kDqk / 16; ++ks) {
          const bf16x8 kf = *(const lds_bf16x8*)(kb[ks & 3] + (ks >> 2) * 1024);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? f32x16{} : s, 0, 0, 0);
          // keep at most a few fragments in flight (bounded register use)
          if ((ks & 1) == 1) __builtin_amdgcn_sched_barrier(0);
        }

        // ---- softmax weights (base 2) ----
        // Lane (col, half) holds, for its query row, keys
        // key0 + 32*mt + 8*r + 4*half + t in s[4*r + t].
        float rmax = kNegInf;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = s[e] * p.scale_log2;
          if (need_mask) {
            const int key = key0 + mt * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            x = key < n_vis_row ? x : kNegInf;
          }
          s[e] = x;
          rmax = fmaxf(rmax, x);
        }
        rmax = wave_max_pair(rmax);
        m_seen = fmaxf(m_seen, rmax);
        if (m_ref == kNegInf) {
          m_ref = rmax;           // nothing accumulated yet: adopt this maximum
        } else if (rmax > m_ref + kRestartThreshold) {
          restart = 1;            // this page is still computed, then thrown away
        }
        const float m_use = m_ref == kNegInf ? 0.f : m_ref;
        float psum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float a = __builtin_amdgcn_exp2f(s[q2 * 8 + e] - m_use);
            const float c = __builtin_amdgcn_exp2f(s[q2 * 8 + e + 1] - m_use);
            psum += a + c;
            w[e >> 1] = pack_bf16x2(a, c);
          }
          pf[q2] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
        l_run += psum;

        // ---- O^T += V^T * P^T : 16 column tiles x 2 k-steps of 16 keys ----
        // k-step kk = 2*mt + q2 covers keys 32*mt + 16*q2 + {4*half + j, 8 + 4*half + j},
        // j = 0..3 (the order in which the S^T accumulator holds them).  Column
        // n = 32*nt + col of such a key sits at vb[nt % 2][j] plus a constant.
#pragma unroll
        for (int nt = 0; nt < kDv / 32; ++nt) {
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            const int krow8 = q2 * 2;   // (first key of the k-step within the half page) / 8
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const int j = e & 3;
              const uint32_t off = ((krow8 + (e >> 2)) * 9 + (nt >> 1)) * 1024;
              const uint16_t lo = *(const lds_u16*)(vb[nt & 1][j] + off);
              const uint16_t hi = *(const lds_u16*)(vb[nt & 1][j + 1] + off);
              w[e >> 1] = (uint32_t)lo | ((uint32_t)hi << 16);
            }
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[q2], acc[nt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }

      ++it;
      if (cur.page + 1 == cur.end)
        done = true;            // leave after the next restart vote
      else
        ++cur.page;
    }
    if (!vote) break;
    // Restart: recompute the segment from its first page with the larger
    // references.  Every wave has passed the vote, so both buffers are free.
    restart = 0;
    m_ref = m_seen;
    cur = seg_start;
    ld = seg_start;
    stage_page(page_ptr(ld), lane_src_off, row_stride_bytes, lds_page[it & 1], wave);
    cursor_next(ld, meta, p.seqlens);
    }

    // ---------------- segment epilogue ----------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = l_tot == 0.f;
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_nat = empty ? kNegInf : (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
    if (row_ok) {
      if (nsplit == 1) {
        uint16_t* op = p.o + ((size_t)(b * p.s_q + q_tok) * p.h_q + q_head) * kDv;
#pragma unroll
        for (int nt = 0; nt < kDv / 32; ++nt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = nt * 32 + r * 8 + half * 4;
            uint2 v;
            v.x = pack_bf16x2(acc[nt][4 * r] * inv, acc[nt][4 * r + 1] * inv);
            v.y = pack_bf16x2(acc[nt][4 * r + 2] * inv, acc[nt][4 * r + 3] * inv);
            *(uint2*)(op + n) = v;
          }
        }
        if (half == 0) p.lse[((size_t)b * p.h_q + q_head) * p.s_q + q_tok] = lse_nat;
      } else {
        float* wp = p.ws_o + ((size_t)(slot * p.h_kv + g) * p.rows + qrow) * kDv;
#pragma unroll
        for (int nt = 0; nt < kDv / 32; ++nt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = nt * 32 + r * 8 + half * 4;
            f32x4 v = {acc[nt][4 * r] * inv, acc[nt][4 * r + 1] * inv, acc[nt][4 * r + 2] * inv,
                       acc[nt][4 * r + 3] * inv};
            *(f32x4*)(wp + n) = v;
          }
        }
        if (half == 0) p.ws_lse[(size_t)(slot * p.h_kv + g) * p.rows + qrow] = lse_nat;
      }
    }

    cursor_next(cur, meta, p.seqlens);
    if (!cur.valid) break;
  }
}

template __global__ void mla_decode_kernel<true>(DecodeParams p);
template __global__ void mla_decode_kernel<false>(DecodeParams p);

}  // namespace mla
