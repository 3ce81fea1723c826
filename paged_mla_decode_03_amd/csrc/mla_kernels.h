// Kernel-side definitions shared by the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;                          // tokens per cache page
constexpr int kDqk = 576;                          // latent row: c^KV (512) + k^R (64)
constexpr int kDv = 512;                           // value width = c^KV
constexpr int kRowsPerBlock = 64;                  // query rows one decode workgroup serves
constexpr int kWaves = 8;                          // 64-lane waves per decode workgroup (2 per SIMD)
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = kDqk * 2;                // 1152 bytes of bf16
constexpr int kChunksPerRow = kRowBytes / 16;      // 72 chunks of 16 bytes
constexpr int kPageBytes = kPage * kRowBytes;      // 73728 bytes staged in LDS per page
constexpr int kPageChunks = kPage * kChunksPerRow; // 4608
constexpr int kNumXcd = 8;                         // MI355X: 8 XCDs, round-robin block dispatch
constexpr int kMetaInts = 8;
constexpr int kMaxWorkers = 4096;
constexpr int kSchedThreads = 256;
constexpr int kCombineThreads = 256;               // wide combine: one 4-wave workgroup per (sequence, head, row)
constexpr int kCombineRowsPerWaveBlock = 4;        // combine: one wave per (sequence, head, query row)

// Wide decode workgroup: 128 query rows of a head, 4 waves (one per SIMD, 512
// registers each), used when a head has more than 128 query rows.  Its two
// page buffers and the softmax weights fill the 160 KB of LDS exactly.
constexpr int kWideRows = 128;
constexpr int kWideWaves = 4;
constexpr int kWideThreads = kWideWaves * 64;
constexpr int kWideDmaPerWave = kPageChunks / 64 / kWideWaves;   // 18
constexpr int kWidePRowBytes = 2 * kPage;                        // unpadded; 16-byte units XOR-swizzled
constexpr int kWidePBytes = kWideRows * kWidePRowBytes;          // 16 KB
static_assert(2 * kPageBytes + kWidePBytes == 160 * 1024, "wide workgroup LDS");

// Query rows one decode workgroup serves for a head with R query rows.
__host__ __device__ constexpr int rows_per_block(int rows) { return rows > kWideRows ? kWideRows : kRowsPerBlock; }

struct DecodeParams {
  const uint16_t* q;            // bf16 [B][s_q][h_q][576]
  const uint16_t* kv;           // bf16 [P][64][h_kv][576]
  const int32_t* block_table;   // [B][max_pages]
  const int32_t* seqlens;       // [B]
  const int32_t* meta;          // [W][8]
  const int32_t* num_splits;    // [B+1]
  uint16_t* o;                  // bf16 [B][s_q][h_q][512]
  float* lse;                   // [B][h_q][s_q]
  float* ws_o;                  // [W+B][h_kv][R][512]
  float* ws_lse;                // [W+B][h_kv][R]
  int batch, s_q, h_q, h_kv;
  int rows;                     // R = s_q * h_q / h_kv
  int group;                    // G = h_q / h_kv
  int max_pages;
  int num_pages;                // pages in the cache (page ids outside [0, num_pages) read as zeros)
  int num_workers;
  int row_blocks;               // ceil(R / rows_per_block(R))
  int causal;
  float scale_log2;             // softmax scale * log2(e) (fp8 cache: times the cache's scale)
  float out_scale;              // factor on the normalised outputs: 1, or the fp8 cache's scale
};

struct CombineParams {
  const int32_t* num_splits;
  const float* ws_o;
  const float* ws_lse;
  uint16_t* o;
  float* lse;
  int batch, s_q, h_q, h_kv, rows, group;
};

struct SchedParams {
  const int32_t* seqlens;
  int32_t* meta;
  int32_t* num_splits;
  int batch;
  int num_workers;
  int fixed_overhead;
};

constexpr int kCheckThreads = 1024;
constexpr int kStreamThreads = 512;
constexpr int kLdsRateBytes = 65536;              // LDS the LDS-rate probe reads
constexpr int kPagesThreads = 1024;

// Whole-page allocator: a stack of free page ids in device memory.
struct PagesParams {
  int32_t* free_pages;          // [num_pages]
  int32_t* state;               // [4]: free count, status of the last call, pages it moved, 0
  int32_t* block_table;         // [B][max_pages]
  const int32_t* seqlens;       // [B]
  const int32_t* release;       // [B] (release only)
  int num_pages, batch, max_pages, s_new;
};

struct CheckParams {
  const int32_t* block_table;   // [B][max_pages]
  const int32_t* seqlens;       // [B]
  int32_t* result;              // [4]
  int batch, max_pages, num_pages;
};

template <bool kSingleHead>
__global__ void mla_decode_kernel(DecodeParams p);
template <bool kSingleHead>
__global__ void mla_decode_fp8_kernel(DecodeParams p);
template <bool kSingleHead>
__global__ void mla_decode_wide_kernel(DecodeParams p);

__global__ void mla_combine_kernel(CombineParams p);
__global__ void mla_combine_wide_kernel(CombineParams p);
__global__ void mla_sched_kernel(SchedParams p);
__global__ void mla_check_kernel(CheckParams p);
__global__ void mla_stream_read_kernel(const uint4* __restrict__ src, size_t n16, uint4* sink);
template <int kKind, int kWavesIn>
__global__ void mla_lds_rate_kernel(int iters, long long* cycles, uint4* sink);
__global__ void mla_pages_init_kernel(PagesParams p);
__global__ void mla_pages_reserve_kernel(PagesParams p);
__global__ void mla_pages_release_kernel(PagesParams p);

}  // namespace mla
