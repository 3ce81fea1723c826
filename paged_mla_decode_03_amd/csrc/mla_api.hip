// Host side of the C ABI declared in include/mla_decode.h: argument checks,
// workspace sizing, launch configuration.  Every check runs before any HIP
// call, so an invalid call launches nothing and needs no device.
#include <math.h>
#include <mutex>

#include <hip/hip_ext.h>

#include "../../include/mla_decode.h"
#include "mla_kernels.h"
#include "mla_append.h"
#include "mla_absorb.h"

namespace {

constexpr int kFixedOverheadPages = 2;   // F of the split rule, in page units

int g_cu_count[64];
std::mutex g_cu_mutex;

int cu_count(int device, int* out) {
  if (device < 0) {
    if (hipGetDevice(&device) != hipSuccess) return MLA_ERR_HIP;
  }
  if (device >= 64) return MLA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[device] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0)
      return MLA_ERR_HIP;
    g_cu_count[device] = n;
  }
  *out = g_cu_count[device];
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Row blocks per head: 64-row workgroups for heads of up to 128 query rows,
// 128-row workgroups above that.
int row_blocks_of(int rows) {
  const int per = mla::rows_per_block(rows);
  return (rows + per - 1) / per;
}

struct Shape {
  int batch, s_q, h_q, h_kv, rows, group;
};

int check_shape(int batch, int s_q, int h_q, int h_kv, int dv, Shape* s) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || h_kv <= 0) return MLA_ERR_INVALID_ARG;
  if (h_q % h_kv != 0) return MLA_ERR_INVALID_ARG;
  if (dv != MLA_D_V) return MLA_ERR_UNSUPPORTED;
  const long long rows = (long long)s_q * (h_q / h_kv);
  if (rows > (1 << 20) || (long long)batch * s_q * h_q > (1LL << 31) / MLA_D_QK) return MLA_ERR_UNSUPPORTED;
  *s = Shape{batch, s_q, h_q, h_kv, (int)rows, h_q / h_kv};
  return MLA_OK;
}

// Workspace layout (each part 256-byte aligned): split partials O [W+B][h_kv][R][512]
// and LSE [W+B][h_kv][R] (fp32).
struct WsLayout {
  size_t lse, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

WsLayout ws_layout(const Shape& s, int num_workers) {
  const size_t slots = (size_t)num_workers + s.batch;
  WsLayout w;
  w.lse = align256(slots * s.h_kv * s.rows * MLA_D_V * 4);
  w.total = w.lse + align256(slots * s.h_kv * s.rows * 4);
  return w;
}

size_t workspace_bytes(const Shape& s, int num_workers) { return ws_layout(s, num_workers).total; }

int check_decode(const void* q, const void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                 int num_pages, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                 int d_qk, int dv, const int32_t* meta, const int32_t* num_splits, int num_workers,
                 int causal, const void* o, const float* lse, const void* workspace,
                 size_t workspace_bytes_given, Shape* s) {
  if (!q || !kvcache || !block_table || !cache_seqlens || !meta || !num_splits || !o || !lse || !workspace)
    return MLA_ERR_INVALID_ARG;
  if (max_pages_per_seq <= 0 || num_pages <= 0 || (causal != 0 && causal != 1)) return MLA_ERR_INVALID_ARG;
  int st = check_shape(batch, s_q, h_q, h_kv, dv, s);
  if (st != MLA_OK) return st;
  if (d_qk != MLA_D_QK) return MLA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(kvcache, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(workspace, 256) || !aligned(block_table, 4) || !aligned(cache_seqlens, 4))
    return MLA_ERR_UNSUPPORTED;
  if ((long long)num_pages * MLA_PAGE_SIZE * h_kv * MLA_D_QK >= (1LL << 40)) return MLA_ERR_UNSUPPORTED;
  if (num_workers <= 0 || num_workers > MLA_MAX_WORKERS) return MLA_ERR_METADATA;
  if (workspace_bytes_given < workspace_bytes(*s, num_workers)) return MLA_ERR_WORKSPACE;
  return MLA_OK;
}

mla::DecodeParams decode_params(const void* q, const void* kvcache, const int32_t* block_table,
                                int max_pages_per_seq, const int32_t* cache_seqlens, const Shape& s,
                                const int32_t* meta, const int32_t* num_splits, int num_workers, int causal,
                                float softmax_scale, void* o, float* lse, void* workspace) {
  mla::DecodeParams p;
  p.q = (const uint16_t*)q;
  p.kv = (const uint16_t*)kvcache;
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.meta = meta;
  p.num_splits = num_splits;
  p.o = (uint16_t*)o;
  p.lse = lse;
  const WsLayout w = ws_layout(s, num_workers);
  char* ws = (char*)workspace;
  p.ws_o = (float*)ws;
  p.ws_lse = (float*)(ws + w.lse);
  p.batch = s.batch;
  p.s_q = s.s_q;
  p.h_q = s.h_q;
  p.h_kv = s.h_kv;
  p.rows = s.rows;
  p.group = s.group;
  p.max_pages = max_pages_per_seq;
  p.num_workers = num_workers;
  p.row_blocks = row_blocks_of(s.rows);
  p.causal = causal;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(192.0f);
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

// With start/stop events, the dispatch itself records them when the kernel
// starts and ends (hipExtLaunchKernelGGL).
template <typename Kernel>
void launch_one(Kernel kernel, int blocks, int threads, const mla::DecodeParams& p, hipStream_t stream,
                hipEvent_t start, hipEvent_t stop) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, stream, start, stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, stream, p);
}

int launch_decode(const mla::DecodeParams& p, hipStream_t stream, hipEvent_t start = nullptr,
                  hipEvent_t stop = nullptr) {
  const int groups = p.num_workers * p.h_kv;
  const int blocks = (groups + mla::kNumXcd - 1) / mla::kNumXcd * mla::kNumXcd * p.row_blocks;
  if (mla::rows_per_block(p.rows) == mla::kWideRows) {
    if (p.h_kv == 1)
      launch_one(mla::mla_decode_wide_kernel<true>, blocks, mla::kWideThreads, p, stream, start, stop);
    else
      launch_one(mla::mla_decode_wide_kernel<false>, blocks, mla::kWideThreads, p, stream, start, stop);
  } else if (p.h_kv == 1) {
    launch_one(mla::mla_decode_kernel<true>, blocks, mla::kThreads, p, stream, start, stop);
  } else {
    launch_one(mla::mla_decode_kernel<false>, blocks, mla::kThreads, p, stream, start, stop);
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_combine(const mla::DecodeParams& d, hipStream_t stream) {
  mla::CombineParams p;
  p.num_splits = d.num_splits;
  p.ws_o = d.ws_o;
  p.ws_lse = d.ws_lse;
  p.o = d.o;
  p.lse = d.lse;
  p.batch = d.batch;
  p.s_q = d.s_q;
  p.h_q = d.h_q;
  p.h_kv = d.h_kv;
  p.rows = d.rows;
  p.group = d.group;
  const long long tasks = (long long)d.batch * d.h_kv * d.rows;
  const int blocks = (int)((tasks + mla::kCombineRowsPerBlock - 1) / mla::kCombineRowsPerBlock);
  hipLaunchKernelGGL(mla::mla_combine_kernel, dim3(blocks), dim3(mla::kCombineRowsPerBlock * 64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int check_append(const void* kv_new, const void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                 int num_pages, const int32_t* cache_seqlens, int batch, int s_new, int h_kv, int d_qk,
                 const int32_t* bad_rows) {
  if (!kv_new || !kvcache || !block_table || !cache_seqlens) return MLA_ERR_INVALID_ARG;
  if (batch <= 0 || s_new <= 0 || h_kv <= 0 || max_pages_per_seq <= 0 || num_pages <= 0) return MLA_ERR_INVALID_ARG;
  if (d_qk != MLA_D_QK) return MLA_ERR_UNSUPPORTED;
  if (!aligned(kv_new, 16) || !aligned(kvcache, 16) || !aligned(block_table, 4) || !aligned(cache_seqlens, 4) ||
      !aligned(bad_rows, 4))
    return MLA_ERR_UNSUPPORTED;
  if ((long long)batch * s_new * h_kv * mla::kChunksPerRow >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
  if ((long long)num_pages * MLA_PAGE_SIZE * h_kv * MLA_D_QK >= (1LL << 40)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer or invalid size";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: unsupported size, alignment or limit";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_METADATA: return "MLA_ERR_METADATA: num_workers out of range";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

int mla_sched_fixed_overhead(void) { return kFixedOverheadPages; }

int mla_num_workers(int device, int rows_per_kv, int h_kv, int* num_workers) {
  if (!num_workers || rows_per_kv <= 0 || h_kv <= 0) return MLA_ERR_INVALID_ARG;
  int cus = 0;
  const int st = cu_count(device, &cus);
  if (st != MLA_OK) return st;
  long long w = cus / ((long long)h_kv * row_blocks_of(rows_per_kv));
  if (w < 1) w = 1;
  if (w > MLA_MAX_WORKERS) w = MLA_MAX_WORKERS;
  *num_workers = (int)w;
  return MLA_OK;
}

int mla_get_metadata(const int32_t* cache_seqlens, int batch, int rows_per_kv, int h_kv, int num_workers,
                     int32_t* tile_scheduler_metadata, int32_t* num_splits, void* stream) {
  if (!cache_seqlens || !tile_scheduler_metadata || !num_splits) return MLA_ERR_INVALID_ARG;
  if (batch <= 0 || rows_per_kv <= 0 || h_kv <= 0) return MLA_ERR_INVALID_ARG;
  if (num_workers <= 0 || num_workers > MLA_MAX_WORKERS) return MLA_ERR_METADATA;
  if (!aligned(cache_seqlens, 4) || !aligned(tile_scheduler_metadata, 4) || !aligned(num_splits, 4))
    return MLA_ERR_UNSUPPORTED;
  mla::SchedParams p;
  p.seqlens = cache_seqlens;
  p.meta = tile_scheduler_metadata;
  p.num_splits = num_splits;
  p.batch = batch;
  p.num_workers = num_workers;
  p.fixed_overhead = kFixedOverheadPages;
  hipLaunchKernelGGL(mla::mla_sched_kernel, dim3(1), dim3(mla::kSchedThreads), 0, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_workspace_bytes(int batch, int s_q, int h_q, int h_kv, int dv, int num_workers) {
  Shape s;
  if (check_shape(batch, s_q, h_q, h_kv, dv, &s) != MLA_OK) return 0;
  if (num_workers <= 0 || num_workers > MLA_MAX_WORKERS) return 0;
  return workspace_bytes(s, num_workers);
}

int mla_decode_splitkv(const void* q, const void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                       int num_pages, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                       int d_qk, int dv, const int32_t* meta, const int32_t* num_splits, int num_workers,
                       int causal, float softmax_scale, void* o, float* lse, void* workspace,
                       size_t workspace_bytes_given, void* stream) {
  Shape s;
  int st = check_decode(q, kvcache, block_table, max_pages_per_seq, num_pages, cache_seqlens, batch, s_q, h_q,
                        h_kv, d_qk, dv, meta, num_splits, num_workers, causal, o, lse, workspace,
                        workspace_bytes_given, &s);
  if (st != MLA_OK) return st;
  const mla::DecodeParams p = decode_params(q, kvcache, block_table, max_pages_per_seq, cache_seqlens, s, meta,
                                            num_splits, num_workers, causal, softmax_scale, o, lse, workspace);
  return launch_decode(p, (hipStream_t)stream);
}

int mla_decode_splitkv_timed(const void* q, const void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                             int num_pages, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                             int d_qk, int dv, const int32_t* meta, const int32_t* num_splits, int num_workers,
                             int causal, float softmax_scale, void* o, float* lse, void* workspace,
                             size_t workspace_bytes_given, void* stream, void* start_event, void* stop_event) {
  Shape s;
  int st = check_decode(q, kvcache, block_table, max_pages_per_seq, num_pages, cache_seqlens, batch, s_q, h_q,
                        h_kv, d_qk, dv, meta, num_splits, num_workers, causal, o, lse, workspace,
                        workspace_bytes_given, &s);
  if (st != MLA_OK) return st;
  if (!start_event || !stop_event) return MLA_ERR_INVALID_ARG;
  const mla::DecodeParams p = decode_params(q, kvcache, block_table, max_pages_per_seq, cache_seqlens, s, meta,
                                            num_splits, num_workers, causal, softmax_scale, o, lse, workspace);
  return launch_decode(p, (hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event);
}

int mla_combine_splits(const int32_t* num_splits, int batch, int s_q, int h_q, int h_kv, int dv,
                       int num_workers, void* o, float* lse, const void* workspace, size_t workspace_bytes_given,
                       void* stream) {
  if (!num_splits || !o || !lse || !workspace) return MLA_ERR_INVALID_ARG;
  Shape s;
  int st = check_shape(batch, s_q, h_q, h_kv, dv, &s);
  if (st != MLA_OK) return st;
  if (num_workers <= 0 || num_workers > MLA_MAX_WORKERS) return MLA_ERR_METADATA;
  if (!aligned(o, 16) || !aligned(lse, 4) || !aligned(workspace, 256)) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes_given < workspace_bytes(s, num_workers)) return MLA_ERR_WORKSPACE;
  mla::DecodeParams d = decode_params(nullptr, nullptr, nullptr, 1, nullptr, s, nullptr, num_splits,
                                      num_workers, 0, 0.f, o, lse, (void*)workspace);
  return launch_combine(d, (hipStream_t)stream);
}

int mla_decode_paged(const void* q, const void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                     int num_pages, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                     int d_qk, int dv, const int32_t* meta, const int32_t* num_splits, int num_workers,
                     int causal, float softmax_scale, void* o, float* lse, void* workspace,
                     size_t workspace_bytes_given, void* stream) {
  Shape s;
  int st = check_decode(q, kvcache, block_table, max_pages_per_seq, num_pages, cache_seqlens, batch, s_q, h_q,
                        h_kv, d_qk, dv, meta, num_splits, num_workers, causal, o, lse, workspace,
                        workspace_bytes_given, &s);
  if (st != MLA_OK) return st;
  const mla::DecodeParams p = decode_params(q, kvcache, block_table, max_pages_per_seq, cache_seqlens, s, meta,
                                            num_splits, num_workers, causal, softmax_scale, o, lse, workspace);
  st = launch_decode(p, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  return launch_combine(p, (hipStream_t)stream);
}

int mla_kvcache_append(const void* kv_new, void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                       int num_pages, const int32_t* cache_seqlens, int batch, int s_new, int h_kv, int d_qk,
                       int32_t* bad_rows, void* stream) {
  const int st = check_append(kv_new, kvcache, block_table, max_pages_per_seq, num_pages, cache_seqlens, batch,
                              s_new, h_kv, d_qk, bad_rows);
  if (st != MLA_OK) return st;
  mla::AppendParams p;
  p.kv_new = (const uint16_t*)kv_new;
  p.kv = (uint16_t*)kvcache;
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.bad_rows = bad_rows;
  p.batch = batch;
  p.s_new = s_new;
  p.h_kv = h_kv;
  p.max_pages = max_pages_per_seq;
  p.num_pages = num_pages;
  p.chunks = batch * s_new * h_kv * mla::kChunksPerRow;
  const int blocks = (p.chunks + mla::kAppendThreads - 1) / mla::kAppendThreads;
  hipLaunchKernelGGL(mla::mla_append_kernel, dim3(blocks), dim3(mla::kAppendThreads), 0, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

namespace {

int launch_absorb(const mla::AbsorbParams& p, bool query, hipStream_t stream) {
  const int n = query ? 512 : mla::kDh;
  const dim3 grid(p.H, n / mla::kAbsorbTileN, (p.T + mla::kAbsorbTileT - 1) / mla::kAbsorbTileT);
  if (query)
    hipLaunchKernelGGL((mla::mla_absorb_kernel<mla::kDh, 512>), grid, dim3(mla::kAbsorbThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((mla::mla_absorb_kernel<512, mla::kDh>), grid, dim3(mla::kAbsorbThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int check_absorb_sizes(int tokens, int h_q) {
  if (tokens <= 0 || h_q <= 0) return MLA_ERR_INVALID_ARG;
  if ((long long)tokens * h_q * MLA_D_QK >= (1LL << 31) || h_q > 65535 ||
      (tokens + mla::kAbsorbTileT - 1) / mla::kAbsorbTileT > 65535)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace

int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk_t, void* q_out, int tokens, int h_q,
                 void* stream) {
  if (!q_nope || !q_rope || !w_uk_t || !q_out) return MLA_ERR_INVALID_ARG;
  const int st = check_absorb_sizes(tokens, h_q);
  if (st != MLA_OK) return st;
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk_t, 16) || !aligned(q_out, 16))
    return MLA_ERR_UNSUPPORTED;
  mla::AbsorbParams p;
  p.a = (const uint16_t*)q_nope;
  p.bt = (const uint16_t*)w_uk_t;
  p.c = (uint16_t*)q_out;
  p.rope = (const uint16_t*)q_rope;
  p.T = tokens;
  p.H = h_q;
  p.a_t = (long long)h_q * mla::kDh;
  p.c_t = (long long)h_q * MLA_D_QK;
  p.c_h = MLA_D_QK;
  return launch_absorb(p, true, (hipStream_t)stream);
}

int mla_absorb_o(const void* o_latent, const void* w_uv, void* out, int tokens, int h_q, void* stream) {
  if (!o_latent || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  const int st = check_absorb_sizes(tokens, h_q);
  if (st != MLA_OK) return st;
  if (!aligned(o_latent, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_UNSUPPORTED;
  mla::AbsorbParams p;
  p.a = (const uint16_t*)o_latent;
  p.bt = (const uint16_t*)w_uv;
  p.c = (uint16_t*)out;
  p.rope = nullptr;
  p.T = tokens;
  p.H = h_q;
  p.a_t = (long long)h_q * MLA_D_V;
  p.c_t = (long long)h_q * mla::kDh;
  p.c_h = mla::kDh;
  return launch_absorb(p, false, (hipStream_t)stream);
}

}  // extern "C"
