// Split-KV tile scheduler for paged MLA decode (gfx950).
//
// The call and its two outputs follow the usage on the dolphin-ai.jp FlashMLA
// page ("FlashMLA の使用方法", step 3); the goal, balancing variable-length
// sequences over the whole chip, is the dynamic load balancing of the
// deepseek.csdn.net article, section 4.2(2).  The split rule itself is this
// library's own:
//
//   n_b pages = ceil(L_b / 64).  On one cost line each sequence takes
//   H = floor(F/2) overhead units (its query load), its n_b page units, then
//   F - H overhead units (its output write); T = sum_b (F + n_b), quota
//   Q = max(1, ceil(T / W)).  Worker w owns units [w*Q, (w+1)*Q) and
//   processes the pages that fall in that range.  With the overhead on both
//   sides of the pages, two workers that share a sequence are each charged
//   one of the fixed costs that every split pays.
//
// Sequence b's pages start at unit s_b + H (s_b = exclusive prefix sum of the
// costs), so the workers meeting them are wf = (s_b+H)/Q .. wl = (s_b+H+n_b-1)/Q,
// and b has wl - wf + 1 splits.  A worker's first segment is the sequence with
// the smallest b that meets it, its last the largest.  Only b's two end
// workers wf and wl can meet other sequences (a worker strictly between them
// lies inside b's pages), so min/max over b are found with LDS atomics at
// those two, which makes the result independent of thread order, and the
// interior workers' rows are written without a lookup (one thread per
// sequence walks its workers, or, for a sequence split more than eight ways,
// its whole wave: plain stores, not dependent LDS reads).
//
// One workgroup, no host synchronisation: the kernel runs on the stream after
// whatever wrote cache_seqlens.
#include "mla_kernels.h"

namespace mla {

namespace {

// Exclusive scan over one value per thread of the workgroup; `total` gets the
// sum.  Each wave scans its 64 values with lane shifts, the waves' totals
// meet in LDS, and every thread adds those of the waves before it: two
// barriers a scan.
__device__ long long block_exclusive_scan(long long v, long long* tmp, long long& total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  long long x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  long long before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kSchedThreads / 64; ++w) {
    const long long t = tmp[w];
    before += w < wave ? t : 0;
    sum += t;
  }
  total = sum;
  __syncthreads();   // tmp is rewritten by the next scan
  return before + x - v;
}

// Pages of a sequence of `seqlen` tokens (0 for seqlen <= 0; no overflow
// near INT_MAX).
__device__ inline int pages_of(int seqlen) { return seqlen > 0 ? (seqlen - 1) / kPage + 1 : 0; }

}  // namespace

__global__ __launch_bounds__(kSchedThreads) void mla_sched_kernel(SchedParams p) {
  __shared__ long long scan_tmp[kSchedThreads];
  __shared__ int first_seq[kMaxWorkers];
  __shared__ int last_seq[kMaxWorkers];
  const int tid = threadIdx.x;
  const int B = p.batch, W = p.num_workers, F = p.fixed_overhead, H = F / 2;

  for (int w = tid; w < W; w += kSchedThreads) {
    first_seq[w] = 0x7fffffff;
    last_seq[w] = -1;
  }

  // Page counts, read once for the first kSchedThreads sequences (every
  // sequence of a batch that fits the workgroup) and again per later chunk.
  const int n0 = tid < B ? pages_of(p.seqlens[tid]) : 0;
  auto pages_at = [&](int base) __attribute__((always_inline)) {
    const int b = base + tid;
    return base == 0 ? n0 : (b < B ? pages_of(p.seqlens[b]) : 0);
  };

  // Total cost T and quota Q.
  long long T = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    const long long cost = b < B ? (long long)F + pages_at(base) : 0;
    long long chunk_total;
    block_exclusive_scan(cost, scan_tmp, chunk_total);
    T += chunk_total;
  }
  const long long Q = T > 0 ? (T + W - 1) / W : 1;

  // Split counts -> num_splits; which workers each sequence meets.
  long long start_carry = 0, split_carry = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    const int n = pages_at(base);
    long long chunk_cost, chunk_splits;
    const long long s_b = start_carry + block_exclusive_scan(b < B ? (long long)F + n : 0, scan_tmp, chunk_cost);
    const long long first_unit = s_b + H;
    long long wf = 0, wl = -1;
    if (n > 0) {
      wf = first_unit / Q;
      wl = (first_unit + n - 1) / Q;
    }
    const long long cnt = n > 0 ? wl - wf + 1 : 0;
    const long long before = split_carry + block_exclusive_scan(cnt, scan_tmp, chunk_splits);
    if (b < B) p.num_splits[b] = (int32_t)before;
    // A worker strictly between wf and wl lies inside b's pages, so b is its
    // only sequence: only the two end workers are contested.  The interior
    // ones are written directly below.
    if (n > 0) {
      atomicMin(&first_seq[wf], b);
      atomicMax(&last_seq[wf], b);
      atomicMin(&first_seq[wl], b);
      atomicMax(&last_seq[wl], b);
    }
    start_carry += chunk_cost;
    split_carry += chunk_splits;
  }
  if (tid == 0) p.num_splits[B] = (int32_t)split_carry;
  __syncthreads();

  // Metadata rows.
  for (int w = tid; w < W; w += kSchedThreads) {
    int32_t* row = p.meta + (size_t)w * kMetaInts;
    if (first_seq[w] == 0x7fffffff) {
      row[0] = 0; row[1] = 0; row[2] = -1; row[3] = 0; row[4] = 0;
    }
    row[5] = 0; row[6] = 0; row[7] = 0;
  }
  // Row of worker w for sequence b (pages from unit first_unit, n of them,
  // workers wf..wl).
  auto write_row = [&](long long w, int b, long long first_unit, int n, long long wf, long long wl)
      __attribute__((always_inline)) {
    int32_t* row = p.meta + (size_t)w * kMetaInts;
    const bool interior = w > wf && w < wl;
    if (interior || first_seq[w] == b) {
      const long long lo = w * Q - first_unit;
      row[0] = b;
      row[1] = (int32_t)(lo > 0 ? lo : 0);
      row[4] = (int32_t)(w - wf);
    }
    if (interior || last_seq[w] == b) {
      const long long hi = (w + 1) * Q - first_unit;
      row[2] = b;
      row[3] = (int32_t)(hi < n ? hi : n);
    }
  };
  const int lane = tid & 63;
  start_carry = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    const int n = pages_at(base);
    long long chunk_cost;
    const long long s_b = start_carry + block_exclusive_scan(b < B ? (long long)F + n : 0, scan_tmp, chunk_cost);
    start_carry += chunk_cost;
    const long long first_unit = s_b + H;
    const long long wf = n > 0 ? first_unit / Q : 0, wl = n > 0 ? (first_unit + n - 1) / Q : -1;
    // A sequence over a few workers walks them alone; one over more than
    // kWalkAlone is walked by its whole wave, 64 workers at a time, so a
    // sequence split a hundred ways costs two passes, not a hundred.
    constexpr long long kWalkAlone = 8;
    const bool shared = wl - wf >= kWalkAlone;
    if (!shared)
      for (long long w = wf; w <= wl; ++w) write_row(w, b, first_unit, n, wf, wl);
    unsigned long long todo = __ballot(shared);
    while (todo) {
      const int src = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int b_s = __shfl(b, src);
      const int n_s = __shfl(n, src);
      const long long fu_s = __shfl(first_unit, src);
      const long long wf_s = __shfl(wf, src), wl_s = __shfl(wl, src);
      for (long long w = wf_s + lane; w <= wl_s; w += 64) write_row(w, b_s, fu_s, n_s, wf_s, wl_s);
    }
  }
}

}  // namespace mla
