// Block write (pa_write_kv) and batched block copy (pa_copy_blocks) — the
// first and third of the three custom kernels named in the vLLM encyclopedia
// entry (tonho.wtf), section "o que isso custou".  Pure data movement: element
// bits are moved, never converted.
#include "pa_kv_store.h"

namespace pa {

// One thread per 16-byte vector of one (token, head): the K vector lands as a
// single 16-byte store in the token's row of a K slab; the V vector's x
// elements are scattered to x consecutive V slab rows (dims), position t % x
// (store_token_vec).  E is the element storage type.
template <typename E>
__global__ __launch_bounds__(256) void write_kv_kernel(const E* __restrict__ k_new,
                                                       const E* __restrict__ v_new,
                                                       E* __restrict__ kc, E* __restrict__ vc,
                                                       const int64_t* __restrict__ slots,
                                                       int64_t num_tokens, int64_t num_slots,
                                                       int H, int D, int BS) {
  constexpr int X = 16 / sizeof(E);
  const int nvec = D / X;
  const int64_t total = num_tokens * H * nvec;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int jv = static_cast<int>(idx % nvec);
    const int64_t th = idx / nvec;
    const int h = static_cast<int>(th % H);
    const int64_t t = th / H;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    store_token_vec<E>(k_new, v_new, kc, vc, t, h, jv, slot, H, D, BS);
  }
}

// Vectors each thread of copy_blocks_kernel has in flight: its loads are all
// issued before its stores, so a copy of a few blocks takes about one memory
// round trip instead of one per vector.
constexpr int kCopyUnroll = 4;

// grid (chunks, num_pairs, 2): z selects the K or the V cache; each thread
// copies kCopyUnroll 16-byte vectors of one block per round, strided by the
// chunk grid.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ kc,
                                                          u32x4* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t vecs_per_block) {
  const int pi = blockIdx.y;
  const int32_t src = pairs[2 * pi];
  const int32_t dst = pairs[2 * pi + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  u32x4* base = blockIdx.z ? vc : kc;
  const u32x4* from = base + src * vecs_per_block;
  u32x4* to = base + dst * vecs_per_block;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i0 < vecs_per_block; i0 += kCopyUnroll * stride) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < vecs_per_block) x[u] = from[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < vecs_per_block) to[i] = x[u];
    }
  }
}

// Whole-block copies between two caches of the same geometry (device memory
// or pinned host memory reached through its device mapping): grid (chunks,
// pairs, 2), z = 0 for K, 1 for V.  Pairs outside either cache are skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const u32x4* __restrict__ src_k, const u32x4* __restrict__ src_v, u32x4* __restrict__ dst_k,
    u32x4* __restrict__ dst_v, const int32_t* __restrict__ pairs, int src_blocks, int dst_blocks,
    int64_t vecs_per_block) {
  const int pi = blockIdx.y;
  const int32_t src = pairs[2 * pi];
  const int32_t dst = pairs[2 * pi + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const u32x4* from = (blockIdx.z ? src_v : src_k) + src * vecs_per_block;
  u32x4* to = (blockIdx.z ? dst_v : dst_k) + dst * vecs_per_block;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < vecs_per_block;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    to[i] = from[i];
}

// Read-rate probe (a measurement helper, not part of the decode): each wave
// reads whole tiles, four at a time (tiles wave, wave + nwaves, ... of the
// order array), with 16-byte loads, non-temporal when NT, and XORs what it
// read; the wave's XOR lands in partials[wave].  The grid is fixed at
// kProbeGroups work-groups of 4 waves.
constexpr int kProbeGroups = 2048;
constexpr int kProbeWaves = kProbeGroups * 4;

template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ buf,
                                                         int64_t num_tiles, int tile_vecs,
                                                         const int32_t* __restrict__ order,
                                                         u32x4* __restrict__ partials) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = __builtin_amdgcn_readfirstlane(
      static_cast<int>((static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6));
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = wave; i < num_tiles; i += 4 * nwaves) {
    int64_t base[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t k = i + u * nwaves;
      const int32_t t = k < num_tiles ? order[k] : -1;
      base[u] = t >= 0 && t < num_tiles ? static_cast<int64_t>(t) * tile_vecs : -1;
    }
#pragma unroll 4
    for (int v = lane; v < tile_vecs; v += 64) {
      u32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = u32x4{0u, 0u, 0u, 0u};
        if (base[u] >= 0) {
          if constexpr (NT)
            x[u] = __builtin_nontemporal_load(buf + base[u] + v);
          else
            x[u] = buf[base[u] + v];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc ^= x[u];
    }
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc[e] ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc[e]), mask, 64));
  if (lane == 0) partials[wave] = acc;
}

// Device-side address of a cache or pair array: device memory as is, pinned
// host memory through its device mapping; nullptr for anything else.
void* device_view(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice) return const_cast<void*>(p);
  if (a.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return d;
  }
  return nullptr;
}

}  // namespace pa

using namespace pa;

PA_EXPORT pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                int num_blocks, int num_kv_heads, int head_dim, int block_size,
                                int dtype, void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t nvec = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim * e / 16);
  const int threads = 256;
  const int64_t want = (nvec + threads - 1) / threads;
  const int blocks = static_cast<int>(want < 65536 ? want : 65536);
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  if (e == 2) {
    hipLaunchKernelGGL(write_kv_kernel<uint16_t>, dim3(blocks), dim3(threads), 0, st,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       slot_mapping, static_cast<int64_t>(num_tokens), num_slots, num_kv_heads,
                       head_dim, block_size);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<uint32_t>, dim3(blocks), dim3(threads), 0, st,
                       static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new),
                       static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                       slot_mapping, static_cast<int64_t>(num_tokens), num_slots, num_kv_heads,
                       head_dim, block_size);
  }
  return launch_status();
}

PA_EXPORT pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                                   int num_pairs, int num_blocks, int num_kv_heads, int head_dim,
                                   int block_size, int dtype, void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID;
  if (num_pairs > 65535) return PA_ERR_INVALID;
  const int64_t vecs = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * e / 16;
  const int threads = 256;
  int64_t chunks = (vecs + threads * kCopyUnroll - 1) / (threads * kCopyUnroll);
  if (chunks < 1) chunks = 1;
  if (chunks > 1024) chunks = 1024;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(chunks), num_pairs, 2),
                     dim3(threads), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), pairs,
                     num_blocks, vecs);
  return launch_status();
}

PA_EXPORT pa_status pa_swap_blocks(const void* src_k, const void* src_v, int src_blocks,
                                   void* dst_k, void* dst_v, int dst_blocks,
                                   const int32_t* pairs, int num_pairs, int num_kv_heads,
                                   int head_dim, int block_size, int dtype, void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0 || num_kv_heads <= 0)
    return PA_ERR_INVALID;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_INVALID;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return PA_ERR_INVALID;
  if (num_pairs > 65535) return PA_ERR_INVALID;
  const void* sk = device_view(src_k);
  const void* sv = device_view(src_v);
  void* dk = device_view(dst_k);
  void* dv = device_view(dst_v);
  const void* pp = device_view(pairs);
  if (!sk || !sv || !dk || !dv || !pp) return PA_ERR_INVALID;
  const int64_t vecs = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * e / 16;
  const int threads = 256;
  int64_t chunks = (vecs + threads * 4 - 1) / (threads * 4);
  if (chunks < 1) chunks = 1;
  if (chunks > 1024) chunks = 1024;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(static_cast<unsigned>(chunks), num_pairs, 2),
                     dim3(threads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(sk), static_cast<const u32x4*>(sv),
                     static_cast<u32x4*>(dk), static_cast<u32x4*>(dv),
                     static_cast<const int32_t*>(pp), src_blocks, dst_blocks, vecs);
  return launch_status();
}

PA_EXPORT int pa_read_probe_partials(void) { return kProbeWaves; }

PA_EXPORT pa_status pa_read_probe(const void* buf, int64_t num_tiles, int tile_bytes,
                                  const int32_t* tile_order, int nontemporal, void* partials,
                                  void* stream) {
  if (num_tiles < 0 || num_tiles > INT32_MAX || tile_bytes <= 0 || tile_bytes % 1024 != 0)
    return PA_ERR_INVALID;
  if (!partials || !aligned16(partials)) return PA_ERR_INVALID;
  if (num_tiles > 0 && (!buf || !tile_order || !aligned16(buf))) return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(kProbeGroups), dim3(256), 0, st,
                       static_cast<const u32x4*>(buf), num_tiles, tile_bytes / 16, tile_order,
                       static_cast<u32x4*>(partials));
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(kProbeGroups), dim3(256), 0, st,
                       static_cast<const u32x4*>(buf), num_tiles, tile_bytes / 16, tile_order,
                       static_cast<u32x4*>(partials));
  return launch_status();
}
