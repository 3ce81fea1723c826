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
// the smallest b that meets it, its last the largest; min/max over b are
// found with LDS atomics, which makes the result independent of thread order.
//
// One workgroup, no host synchronisation: the kernel runs on the stream after
// whatever wrote cache_seqlens.
#include "mla_kernels.h"

namespace mla {

namespace {

// Exclusive scan over one value per thread of the workgroup; `total` gets the sum.
__device__ long long block_exclusive_scan(long long v, long long* tmp, long long& total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    long long add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  long long incl = tmp[tid];
  total = tmp[kSchedThreads - 1];
  __syncthreads();
  return incl - v;
}

__device__ inline int pages_of(int seqlen) { return (seqlen + kPage - 1) / kPage; }

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

  // Total cost T and quota Q.
  long long T = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    const long long cost = b < B ? (long long)F + pages_of(p.seqlens[b]) : 0;
    long long chunk_total;
    block_exclusive_scan(cost, scan_tmp, chunk_total);
    T += chunk_total;
  }
  const long long Q = T > 0 ? (T + W - 1) / W : 1;

  // Split counts -> num_splits; which workers each sequence meets.
  long long start_carry = 0, split_carry = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    const int n = b < B ? pages_of(p.seqlens[b]) : 0;
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
    for (long long w = wf; w <= wl; ++w) {
      atomicMin(&first_seq[w], b);
      atomicMax(&last_seq[w], b);
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
  start_carry = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    const int n = b < B ? pages_of(p.seqlens[b]) : 0;
    long long chunk_cost;
    const long long s_b = start_carry + block_exclusive_scan(b < B ? (long long)F + n : 0, scan_tmp, chunk_cost);
    start_carry += chunk_cost;
    if (n == 0) continue;
    const long long first_unit = s_b + H;
    const long long wf = first_unit / Q, wl = (first_unit + n - 1) / Q;
    for (long long w = wf; w <= wl; ++w) {
      int32_t* row = p.meta + (size_t)w * kMetaInts;
      if (first_seq[w] == b) {
        const long long lo = w * Q - first_unit;
        row[0] = b;
        row[1] = (int32_t)(lo > 0 ? lo : 0);
        row[4] = (int32_t)(w - wf);
      }
      if (last_seq[w] == b) {
        const long long hi = (w + 1) * Q - first_unit;
        row[2] = b;
        row[3] = (int32_t)(hi < n ? hi : n);
      }
    }
  }
}

}  // namespace mla
