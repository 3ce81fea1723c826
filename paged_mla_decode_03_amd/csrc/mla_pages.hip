// Whole-page allocator for the paged latent cache (gfx950).
//
// Memory is handed out and taken back only in whole pages of 64 token slots
// (the lukefan.com talk on FlashMLA, on allocating and freeing in whole pages
// of 64; deepseek.csdn.net FlashMLA article, section 4.2(2), paged KV cache
// management), so the pool never fragments below a page and a sequence's
// cache is always a whole number of pages mapped through its block_table
// row.  The free pages form a stack, free_pages[0 .. count) with the top at
// count - 1, kept in device memory with the counter, so the allocator runs
// on the stream between decode steps without a host round trip:
//   * reserve: before s_new tokens are appended to every sequence, sequence
//     b needs ceil((L_b + s_new) / 64) - ceil(L_b / 64) more pages; in batch
//     order (an exclusive scan of the needs), and each sequence's blocks in
//     ascending order, they are popped from the top of the stack into its
//     block_table row;
//   * release: the mapped pages of every flagged sequence are pushed back in
//     the same order and its entries set to -1.
// A call that cannot be satisfied changes nothing and leaves its reason in
// state[1]: 1 when the free pages do not suffice (reserve) or the stack
// would overflow (release: pages given back twice), 2 when a length or a
// page id is out of range.  One workgroup: the decision is taken after the
// whole scan, before any write.
#include "mla_kernels.h"

namespace mla {

namespace {

__device__ inline int pages_for(long long tokens) { return tokens > 0 ? (int)((tokens - 1) / kPage + 1) : 0; }

// Exclusive scan over one value per thread; `total` gets the sum.
__device__ long long scan_exclusive(long long v, long long* tmp, long long& total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPagesThreads; off <<= 1) {
    const long long add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const long long incl = tmp[tid];
  total = tmp[kPagesThreads - 1];
  __syncthreads();
  return incl - v;
}

}  // namespace

__global__ __launch_bounds__(256) void mla_pages_init_kernel(PagesParams p) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < p.num_pages; i += (long long)gridDim.x * 256)
    p.free_pages[i] = (int32_t)(p.num_pages - 1 - i);
  if (blockIdx.x == 0 && threadIdx.x < 4) p.state[threadIdx.x] = threadIdx.x == 0 ? p.num_pages : 0;
}

__global__ __launch_bounds__(kPagesThreads) void mla_pages_reserve_kernel(PagesParams p) {
  __shared__ long long tmp[kPagesThreads];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int count = p.state[0];
  if (tid == 0) bad = 0;
  __syncthreads();
  // Needs and their total; lengths past the table row are refused.
  long long total = 0;
  for (int base = 0; base < p.batch; base += kPagesThreads) {
    const int b = base + tid;
    long long need = 0;
    if (b < p.batch) {
      const long long L = p.seqlens[b];
      const int want = pages_for(L + p.s_new);
      if (L < 0 || want > p.max_pages) atomicOr(&bad, 1);
      else need = want - pages_for(L);
    }
    long long chunk;
    scan_exclusive(need, tmp, chunk);
    total += chunk;
  }
  const bool refuse_range = bad != 0;
  const bool refuse_space = !refuse_range && total > count;
  if (!refuse_range && !refuse_space) {
    long long carry = 0;
    for (int base = 0; base < p.batch; base += kPagesThreads) {
      const int b = base + tid;
      int have = 0, want = 0;
      if (b < p.batch) {
        const long long L = p.seqlens[b];
        have = pages_for(L);
        want = pages_for(L + p.s_new);
      }
      long long chunk;
      const long long off = carry + scan_exclusive(want - have, tmp, chunk);
      for (int j = have; j < want; ++j)
        p.block_table[(size_t)b * p.max_pages + j] = p.free_pages[count - 1 - (off + (j - have))];
      carry += chunk;
    }
  }
  __syncthreads();   // every thread has read state[0] and the stack
  if (tid == 0) {
    if (!refuse_range && !refuse_space) p.state[0] = (int32_t)(count - total);
    p.state[1] = refuse_range ? 2 : (refuse_space ? 1 : 0);
    p.state[2] = refuse_range ? 0 : (int32_t)total;
    p.state[3] = 0;
  }
}

__global__ __launch_bounds__(kPagesThreads) void mla_pages_release_kernel(PagesParams p) {
  __shared__ long long tmp[kPagesThreads];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int count = p.state[0];
  if (tid == 0) bad = 0;
  __syncthreads();
  long long total = 0;
  for (int base = 0; base < p.batch; base += kPagesThreads) {
    const int b = base + tid;
    long long n = 0;
    if (b < p.batch && p.release[b] != 0) {
      const long long L = p.seqlens[b];
      const int np = pages_for(L);
      if (L < 0 || np > p.max_pages) {
        atomicOr(&bad, 1);
      } else {
        for (int j = 0; j < np; ++j) {
          const int pid = p.block_table[(size_t)b * p.max_pages + j];
          if (pid < 0 || pid >= p.num_pages) atomicOr(&bad, 1);
        }
        n = np;
      }
    }
    long long chunk;
    scan_exclusive(n, tmp, chunk);
    total += chunk;
  }
  const bool refuse_range = bad != 0;
  const bool refuse_space = !refuse_range && count + total > p.num_pages;
  if (!refuse_range && !refuse_space) {
    long long carry = 0;
    for (int base = 0; base < p.batch; base += kPagesThreads) {
      const int b = base + tid;
      const int n = (b < p.batch && p.release[b] != 0) ? pages_for(p.seqlens[b]) : 0;
      long long chunk;
      const long long off = carry + scan_exclusive(n, tmp, chunk);
      for (int j = 0; j < n; ++j) {
        int32_t* e = p.block_table + (size_t)b * p.max_pages + j;
        p.free_pages[count + off + j] = *e;
        *e = -1;
      }
      carry += chunk;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (!refuse_range && !refuse_space) p.state[0] = (int32_t)(count + total);
    p.state[1] = refuse_range ? 2 : (refuse_space ? 1 : 0);
    p.state[2] = refuse_range ? 0 : (int32_t)total;
    p.state[3] = 0;
  }
}

}  // namespace mla
