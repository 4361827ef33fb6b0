// One decode iteration as the central KV-cache manager hands it to the GPU
// (vLLM encyclopedia entry, tonho.wtf, section "como funciona": the manager
// ships the block tables with each iteration's input).  Host side: pool
// append, tables and lengths into one pinned staging buffer; device side: one
// host-to-device copy, then copy-on-write copies, the block write and decode,
// all on the caller's stream.
#include <algorithm>
#include <cstring>
#include <numeric>

#include "pa_internal.h"

extern "C" int64_t pa_pool_shared_blocks(const pa_pool* p);

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct StagingLayout {
  size_t slots, pairs, lens, order, tables, total;
};

StagingLayout staging_layout(int n, int maxb) {
  StagingLayout L;
  L.slots = 0;
  L.pairs = L.slots + align_up(sizeof(int64_t) * n);
  L.lens = L.pairs + align_up(sizeof(int32_t) * 2 * n);
  L.order = L.lens + align_up(sizeof(int32_t) * n);
  L.tables = L.order + align_up(sizeof(int32_t) * n);
  L.total = L.tables + align_up(sizeof(int32_t) * static_cast<size_t>(n) * maxb);
  return L;
}

// Copies the pinned host staging buffer into device memory from a kernel on
// the caller's stream: the compute queue does not wait on a copy engine.
// System-scope loads always see what the host wrote before the launch.
__global__ __launch_bounds__(256) void stage_copy_kernel(const uint64_t* __restrict__ src,
                                                         uint64_t* __restrict__ dst, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

using namespace pa;

PA_EXPORT size_t pa_decode_step_staging_size(int num_seqs, int max_blocks_per_seq) {
  if (num_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
  return staging_layout(num_seqs, max_blocks_per_seq).total;
}

PA_EXPORT pa_status pa_decode_step(pa_pool* pool, const int64_t* seqs, int num_seqs,
                                   const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                                   int block_size, const void* q, void* out, int num_q_heads,
                                   float scale, int partition_size, int max_blocks_per_seq,
                                   void* host_staging, void* dev_staging, size_t staging_bytes,
                                   void* workspace, size_t workspace_bytes, int dtype,
                                   void* stream) {
  if (!pool || num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!seqs || !host_staging || !dev_staging) return PA_ERR_INVALID;
  // everything the device calls would reject is rejected before the pool changes
  if (elem_bytes(dtype) == 0 || !supported_head_dim(head_dim) ||
      !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_blocks <= 0 || partition_size < 0 || partition_size % 32 != 0 ||
      !std::isfinite(scale))
    return PA_ERR_INVALID;
  if (!k_new || !v_new || !k_cache || !v_cache || !q || !out) return PA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(q) || !aligned16(out) || (workspace && !aligned16(workspace)))
    return PA_ERR_INVALID;
  const StagingLayout L = staging_layout(num_seqs, max_blocks_per_seq);
  if (staging_bytes < L.total || !aligned16(host_staging) || !aligned16(dev_staging))
    return PA_ERR_INVALID;
  {
    // capacity: each table after the append fits max_blocks_per_seq; the
    // workspace covers the longest context after the append
    int pre_max = 0;
    for (int i = 0; i < num_seqs; ++i) {
      int nb = 0, nt = 0;
      const pa_status q_st = pa_seq_block_table(pool, seqs[i], nullptr, 0, &nb, &nt);
      if (q_st == PA_ERR_UNKNOWN_SEQ) return q_st;
      const int nb_after = nb + (nt % block_size == 0 ? 1 : 0);
      if (nb_after > max_blocks_per_seq) return PA_ERR_INVALID;
      pre_max = nt + 1 > pre_max ? nt + 1 : pre_max;
    }
    const size_t need =
        pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, pre_max, partition_size);
    if (need > workspace_bytes || (need > 0 && !workspace)) return PA_ERR_INVALID;
  }
  char* h = static_cast<char*>(host_staging);
  char* d = static_cast<char*>(dev_staging);
  int64_t* h_slots = reinterpret_cast<int64_t*>(h + L.slots);
  int32_t* h_pairs = reinterpret_cast<int32_t*>(h + L.pairs);
  int32_t* h_lens = reinterpret_cast<int32_t*>(h + L.lens);
  int32_t* h_order = reinterpret_cast<int32_t*>(h + L.order);
  int32_t* h_tab = reinterpret_cast<int32_t*>(h + L.tables);

  // 1. host pool: one new position per sequence (all-or-nothing)
  int npairs = 0;
  pa_status st = pa_seq_append_batch(pool, seqs, num_seqs, 1, h_slots, h_pairs, &npairs);
  if (st != PA_OK) return st;
  // 2. tables and lengths after the append
  st = pa_pool_block_tables(pool, seqs, num_seqs, h_tab, max_blocks_per_seq, h_lens);
  if (st != PA_OK) return st;
  int max_ctx = 0;
  for (int i = 0; i < num_seqs; ++i) max_ctx = h_lens[i] > max_ctx ? h_lens[i] : max_ctx;
  // sharers together, longest work first
  st = pa_decode_order(h_tab, max_blocks_per_seq, h_lens, num_seqs, h_order);
  if (st != PA_OK) return st;
  const int flags = pa_pool_shared_blocks(pool) > 0 ? PA_DECODE_SHARED_KV : 0;

  // 3. one host-to-device copy of slots, pairs, lengths, order and tables:
  //    a copy kernel reading the pinned buffer when it is mapped on the device,
  //    else an asynchronous copy
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* h_dev = nullptr;
  if (hipHostGetDevicePointer(&h_dev, host_staging, 0) == hipSuccess && h_dev) {
    const int64_t n = static_cast<int64_t>(L.total / sizeof(uint64_t));
    const int blocks = static_cast<int>((n + 255) / 256 < 64 ? (n + 255) / 256 : 64);
    hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint64_t*>(h_dev), reinterpret_cast<uint64_t*>(d), n);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  } else {
    (void)hipGetLastError();
    if (hipMemcpyAsync(d, h, L.total, hipMemcpyHostToDevice, s) != hipSuccess) return PA_ERR_HIP;
  }

  // 4. copy-on-write, block write, decode
  if (npairs > 0) {
    st = pa_copy_blocks(k_cache, v_cache, reinterpret_cast<const int32_t*>(d + L.pairs), npairs,
                        num_blocks, num_kv_heads, head_dim, block_size, dtype, stream);
    if (st != PA_OK) return st;
  }
  st = pa_write_kv(k_new, v_new, k_cache, v_cache, reinterpret_cast<const int64_t*>(d + L.slots),
                   num_seqs, num_blocks, num_kv_heads, head_dim, block_size, dtype, stream);
  if (st != PA_OK) return st;
  return decode_impl(out, q, k_cache, v_cache, reinterpret_cast<const int32_t*>(d + L.tables),
                     max_blocks_per_seq, reinterpret_cast<const int32_t*>(d + L.lens), num_seqs,
                     max_ctx, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     partition_size, workspace, workspace_bytes, dtype, flags,
                     reinterpret_cast<const int32_t*>(d + L.order), stream);
}
