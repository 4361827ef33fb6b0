// One decode iteration as the central KV-cache manager hands it to the GPU
// (vLLM encyclopedia entry, tonho.wtf, section "como funciona": the manager
// ships the block tables with each iteration's input; beam candidates share
// blocks and the sharing changes every step).  Host side: the pool step
// (append, or beam fork / retire / append), tables and lengths into one pinned
// staging buffer; device side, all on the caller's stream: one host-to-device
// copy, copy-on-write copies and the decode, which also stores the step's new
// K/V (fp16 / bf16; fp32 runs the block write before it).
#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

#include "pa_kv_store.h"

extern "C" int64_t pa_pool_shared_blocks(const pa_pool* p);

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct StagingLayout {
  size_t slots, pairs, lens, order, prefix, groups, members, tables, total;
};

StagingLayout staging_layout(int n, int maxb) {
  StagingLayout L;
  L.slots = 0;
  L.pairs = L.slots + align_up(sizeof(int64_t) * n);
  L.lens = L.pairs + align_up(sizeof(int32_t) * 2 * n);
  L.order = L.lens + align_up(sizeof(int32_t) * n);
  L.prefix = L.order + align_up(sizeof(int32_t) * n);
  L.groups = L.prefix + align_up(sizeof(int32_t) * n);
  L.members = L.groups + align_up(sizeof(int32_t) * 3 * n);
  L.tables = L.members + align_up(sizeof(int32_t) * n);
  L.total = L.tables + align_up(sizeof(int32_t) * static_cast<size_t>(n) * maxb);
  return L;
}

// Shared prefixes shorter than this stay on the plain path.
constexpr int kCascadeMinPrefix = 512;

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

namespace {

// The device side of a step, shared by pa_decode_step and
// pa_beam_decode_step.
struct StepDev {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  int num_blocks, num_kv_heads, head_dim, block_size;
  const void* q;
  void* out;
  int num_q_heads;
  float scale;
  int partition_size, max_blocks_per_seq;
  void* host_staging;
  void* dev_staging;
  size_t staging_bytes;
  void* workspace;
  size_t workspace_bytes;
  int dtype;
  void* stream;
};

// Everything the device calls would reject, for n sequences.
pa_status check_dev(const StepDev& a, int n) {
  if (!a.host_staging || !a.dev_staging) return PA_ERR_INVALID;
  if (elem_bytes(a.dtype) == 0 || !supported_head_dim(a.head_dim) ||
      !supported_block_size(a.block_size))
    return PA_ERR_UNSUPPORTED;
  if (n > 65535 || a.num_q_heads > 65535) return PA_ERR_INVALID;  // the decode's grid limits
  if (a.num_q_heads <= 0 || a.num_kv_heads <= 0 || a.num_q_heads % a.num_kv_heads != 0 ||
      a.num_blocks <= 0 || a.partition_size < 0 || a.partition_size % 32 != 0 ||
      !(a.scale > 0.f) || !std::isfinite(a.scale))
    return PA_ERR_INVALID;
  if (!a.k_new || !a.v_new || !a.k_cache || !a.v_cache || !a.q || !a.out) return PA_ERR_INVALID;
  if (!aligned16(a.k_new) || !aligned16(a.v_new) || !aligned16(a.k_cache) ||
      !aligned16(a.v_cache) || !aligned16(a.q) || !aligned16(a.out) ||
      (a.workspace && !aligned16(a.workspace)))
    return PA_ERR_INVALID;
  const StagingLayout L = staging_layout(n, a.max_blocks_per_seq);
  if (a.staging_bytes < L.total || !aligned16(a.host_staging) || !aligned16(a.dev_staging))
    return PA_ERR_INVALID;
  return PA_OK;
}

// Table capacity and workspace for sequences whose context before the step
// is `ctx[i]` over `nb[i]` blocks and grows by one position.
pa_status check_growth(const StepDev& a, int n, const int* nb, const int* ctx) {
  int pre_max = 0;
  for (int i = 0; i < n; ++i) {
    const int nb_after = nb[i] + (ctx[i] % a.block_size == 0 ? 1 : 0);
    if (nb_after > a.max_blocks_per_seq) return PA_ERR_INVALID;
    pre_max = ctx[i] + 1 > pre_max ? ctx[i] + 1 : pre_max;
  }
  const size_t need =
      pa_decode_workspace_size(n, a.num_q_heads, a.head_dim, pre_max, a.partition_size);
  if (need > a.workspace_bytes || (need > 0 && !a.workspace)) return PA_ERR_INVALID;
  return PA_OK;
}

// After the pool has given slots and pairs (already in the staging buffer):
// tables, lengths and issue order into staging, one host-to-device copy, then
// copy-on-write and the decode with its block write on the stream.
pa_status launch_step(pa_pool* pool, const StepDev& a, const int64_t* seqs, int n, int npairs) {
  const StagingLayout L = staging_layout(n, a.max_blocks_per_seq);
  char* h = static_cast<char*>(a.host_staging);
  char* d = static_cast<char*>(a.dev_staging);
  int32_t* h_lens = reinterpret_cast<int32_t*>(h + L.lens);
  int32_t* h_order = reinterpret_cast<int32_t*>(h + L.order);
  int32_t* h_tab = reinterpret_cast<int32_t*>(h + L.tables);
  pa_status st = pa_pool_block_tables(pool, seqs, n, h_tab, a.max_blocks_per_seq, h_lens);
  if (st != PA_OK) return st;
  int max_ctx = 0;
  for (int i = 0; i < n; ++i) max_ctx = h_lens[i] > max_ctx ? h_lens[i] : max_ctx;
  // sharers together, longest work first
  st = pa_decode_order(h_tab, a.max_blocks_per_seq, h_lens, n, h_order);
  if (st != PA_OK) return st;
  const int flags = pa_pool_shared_blocks(pool) > 0 ? PA_DECODE_SHARED_KV : 0;
  // shared prefixes: one prefix pass per group of sequences sharing blocks,
  // when the workspace has room for the cascade's partials
  CascadePlan plan{reinterpret_cast<const int32_t*>(d + L.prefix),
                   reinterpret_cast<const int32_t*>(d + L.groups),
                   reinterpret_cast<const int32_t*>(d + L.members), 0, 0, 0, 0};
  if (flags && a.dtype != PA_F32 &&
      pa_decode_cascade_workspace_size(n, a.num_q_heads, a.head_dim, max_ctx,
                                       a.partition_size) <= a.workspace_bytes &&
      a.workspace) {
    st = pa_cascade_plan(h_tab, a.max_blocks_per_seq, h_lens, n, a.block_size, a.num_q_heads,
                         a.num_kv_heads, kCascadeMinPrefix,
                         reinterpret_cast<int32_t*>(h + L.prefix),
                         reinterpret_cast<int32_t*>(h + L.groups),
                         reinterpret_cast<int32_t*>(h + L.members), &plan.ngroups,
                         &plan.max_prefix, &plan.max_members, &plan.max_rest);
    if (st != PA_OK) return st;
  }

  // the block write rides in the decode (fp16 / bf16): the decode wave that
  // ends a context takes the appended token from k_new / v_new; a shared
  // prefix never reaches the appended position (its block is private)
  bool fused_write = a.dtype != PA_F32;
  if (plan.ngroups > 0) {
    const int32_t* pre = reinterpret_cast<const int32_t*>(h + L.prefix);
    for (int i = 0; i < n && fused_write; ++i) fused_write = pre[i] < h_lens[i];
  }

  // one host-to-device copy of slots, pairs, lengths, order and tables: a
  // copy kernel reading the pinned buffer when it is mapped on the device,
  // else an asynchronous copy
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  void* h_dev = nullptr;
  if (hipHostGetDevicePointer(&h_dev, a.host_staging, 0) == hipSuccess && h_dev) {
    const int64_t nw = static_cast<int64_t>(L.total / sizeof(uint64_t));
    const int blocks = static_cast<int>((nw + 255) / 256 < 64 ? (nw + 255) / 256 : 64);
    hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint64_t*>(h_dev), reinterpret_cast<uint64_t*>(d), nw);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  } else {
    (void)hipGetLastError();
    if (hipMemcpyAsync(d, h, L.total, hipMemcpyHostToDevice, s) != hipSuccess) return PA_ERR_HIP;
  }
  if (npairs > 0) {
    st = pa_copy_blocks(a.k_cache, a.v_cache, reinterpret_cast<const int32_t*>(d + L.pairs),
                        npairs, a.num_blocks, a.num_kv_heads, a.head_dim, a.block_size, a.dtype,
                        a.stream);
    if (st != PA_OK) return st;
  }
  if (!fused_write) {
    st = pa_write_kv(a.k_new, a.v_new, a.k_cache, a.v_cache,
                     reinterpret_cast<const int64_t*>(d + L.slots), n, a.num_blocks,
                     a.num_kv_heads, a.head_dim, a.block_size, a.dtype, a.stream);
    if (st != PA_OK) return st;
  }
  const NewKV nkv{fused_write ? a.k_new : nullptr, fused_write ? a.v_new : nullptr};
  return decode_impl(a.out, a.q, a.k_cache, a.v_cache,
                     reinterpret_cast<const int32_t*>(d + L.tables), a.max_blocks_per_seq,
                     reinterpret_cast<const int32_t*>(d + L.lens), n, max_ctx, a.num_q_heads,
                     a.num_kv_heads, a.head_dim, a.block_size, a.num_blocks, a.scale,
                     a.partition_size, a.workspace, a.workspace_bytes, a.dtype, flags,
                     reinterpret_cast<const int32_t*>(d + L.order), a.stream, &plan, &nkv);
}

}  // namespace

PA_EXPORT pa_status pa_decode_step(pa_pool* pool, const int64_t* seqs, int num_seqs,
                                   const int32_t* tokens, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, int num_blocks,
                                   int num_kv_heads, int head_dim,
                                   int block_size, const void* q, void* out, int num_q_heads,
                                   float scale, int partition_size, int max_blocks_per_seq,
                                   void* host_staging, void* dev_staging, size_t staging_bytes,
                                   void* workspace, size_t workspace_bytes, int dtype,
                                   void* stream) {
  if (!pool || num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!seqs) return PA_ERR_INVALID;
  const StepDev a{k_new, v_new, k_cache, v_cache, num_blocks, num_kv_heads, head_dim,
                  block_size, q, out, num_q_heads, scale, partition_size, max_blocks_per_seq,
                  host_staging, dev_staging, staging_bytes, workspace, workspace_bytes, dtype,
                  stream};
  // everything the device calls would reject is rejected before the pool changes
  pa_status st = check_dev(a, num_seqs);
  if (st != PA_OK) return st;
  std::vector<int> nb(num_seqs), nt(num_seqs);
  for (int i = 0; i < num_seqs; ++i) {
    st = pa_seq_block_table(pool, seqs[i], nullptr, 0, &nb[i], &nt[i]);
    if (st == PA_ERR_UNKNOWN_SEQ) return st;
  }
  st = check_growth(a, num_seqs, nb.data(), nt.data());
  if (st != PA_OK) return st;
  const StagingLayout L = staging_layout(num_seqs, max_blocks_per_seq);
  char* h = static_cast<char*>(host_staging);
  // host pool: one new position per sequence (all-or-nothing); with token
  // ids, sequences a prefix index tracks keep feeding it
  int npairs = 0;
  st = tokens ? pa_seq_append_tokens(pool, seqs, num_seqs, tokens, 1,
                                     reinterpret_cast<int64_t*>(h + L.slots),
                                     reinterpret_cast<int32_t*>(h + L.pairs), &npairs)
              : pa_seq_append_batch(pool, seqs, num_seqs, 1,
                                    reinterpret_cast<int64_t*>(h + L.slots),
                                    reinterpret_cast<int32_t*>(h + L.pairs), &npairs);
  if (st != PA_OK) return st;
  return launch_step(pool, a, seqs, num_seqs, npairs);
}

PA_EXPORT pa_status pa_beam_decode_step(pa_pool* pool, const int64_t* old_beams, int n_old,
                                        const int64_t* parents, const int64_t* new_beams,
                                        int n_new, const int32_t* tokens, const void* k_new,
                                        const void* v_new, void* k_cache, void* v_cache,
                                        int num_blocks,
                                        int num_kv_heads, int head_dim, int block_size,
                                        const void* q, void* out, int num_q_heads, float scale,
                                        int partition_size, int max_blocks_per_seq,
                                        void* host_staging, void* dev_staging,
                                        size_t staging_bytes, void* workspace,
                                        size_t workspace_bytes, int dtype, void* stream) {
  if (!pool || n_old < 0 || n_new < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID;
  if (n_new > 0 && (!parents || !new_beams)) return PA_ERR_INVALID;
  if (n_old > 0 && !old_beams) return PA_ERR_INVALID;
  const StepDev a{k_new, v_new, k_cache, v_cache, num_blocks, num_kv_heads, head_dim,
                  block_size, q, out, num_q_heads, scale, partition_size, max_blocks_per_seq,
                  host_staging, dev_staging, staging_bytes, workspace, workspace_bytes, dtype,
                  stream};
  if (n_new > 0) {
    pa_status st = check_dev(a, n_new);
    if (st != PA_OK) return st;
    std::vector<int> nb(n_new), nt(n_new);
    for (int j = 0; j < n_new; ++j) {
      st = pa_seq_block_table(pool, parents[j], nullptr, 0, &nb[j], &nt[j]);
      if (st == PA_ERR_UNKNOWN_SEQ) return st;
    }
    st = check_growth(a, n_new, nb.data(), nt.data());
    if (st != PA_OK) return st;
  }
  const StagingLayout L = staging_layout(n_new > 0 ? n_new : 1, max_blocks_per_seq);
  char* h = static_cast<char*>(host_staging);
  int npairs = 0;
  pa_status st = pa_seq_beam_step(pool, old_beams, n_old, parents, new_beams, n_new, tokens,
                                  n_new > 0 ? reinterpret_cast<int64_t*>(h + L.slots) : nullptr,
                                  n_new > 0 ? reinterpret_cast<int32_t*>(h + L.pairs) : nullptr,
                                  &npairs);
  if (st != PA_OK || n_new == 0) return st;
  return launch_step(pool, a, new_beams, n_new, npairs);
}
