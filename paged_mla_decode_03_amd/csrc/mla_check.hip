// Input checker for the paged cache's tables (gfx950).
//
// The decode reads block_table and cache_seqlens on the device, so their
// contents cannot be checked by the host before a launch.  The usage on the
// dolphin-ai.jp FlashMLA page ("FlashMLA の使用方法", step 4) passes both
// straight to the kernel; the paging contract (deepseek.csdn.net FlashMLA
// article, section 4.2(1)) is that logical block j of sequence b lives in
// physical page block_table[b][j].  This kernel verifies that contract for
// every block a decode would read:
//   * 0 <= L_b <= 64 * max_pages_per_seq, and
//   * 0 <= block_table[b][j] < num_pages for j < ceil(L_b / 64).
// It writes result[0] = number of bad entries (lengths and page ids),
// result[1] = the first bad sequence (-1 if none), result[2] = its first bad
// block (-1 for a bad length), result[3] = 0.  One workgroup: thread 0
// writes the result after a workgroup reduction, so it needs no
// initialisation.
#include "mla_kernels.h"

namespace mla {

__global__ __launch_bounds__(kCheckThreads) void mla_check_kernel(CheckParams p) {
  __shared__ int bad_count;
  __shared__ unsigned long long first_bad;   // (b << 32) | (block + 1), minimum over threads
  const int tid = threadIdx.x;
  if (tid == 0) {
    bad_count = 0;
    first_bad = ~0ull;
  }
  __syncthreads();
  int count = 0;
  unsigned long long first = ~0ull;
  // One thread per (sequence, block), blocks of a sequence consecutive.
  const long long total = (long long)p.batch * (p.max_pages + 1);
  for (long long i = tid; i < total; i += kCheckThreads) {
    const int b = (int)(i / (p.max_pages + 1));
    const int j = (int)(i - (long long)b * (p.max_pages + 1)) - 1;   // -1: the length itself
    const int L = p.seqlens[b];
    const bool len_ok = L >= 0 && (long long)L <= (long long)kPage * p.max_pages;
    bool bad;
    if (j < 0) {
      bad = !len_ok;
    } else {
      const int n = len_ok ? (L + kPage - 1) / kPage : 0;
      const int pid = j < n ? p.block_table[(size_t)b * p.max_pages + j] : 0;
      bad = j < n && (pid < 0 || pid >= p.num_pages);
    }
    if (bad) {
      ++count;
      const unsigned long long key = ((unsigned long long)b << 32) | (unsigned)(j + 1);
      first = key < first ? key : first;
    }
  }
  if (count) {
    atomicAdd(&bad_count, count);
    atomicMin(&first_bad, first);
  }
  __syncthreads();
  if (tid == 0) {
    const bool any = bad_count != 0;
    p.result[0] = bad_count;
    p.result[1] = any ? (int)(first_bad >> 32) : -1;
    p.result[2] = any ? (int)(first_bad & 0xffffffffu) - 1 : -1;
    p.result[3] = 0;
  }
}

}  // namespace mla
