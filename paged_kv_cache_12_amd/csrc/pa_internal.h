// Internal helpers shared by the HIP translation units of libpa.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/pa.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

inline int elem_bytes(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16:
    case PA_BF16: return 2;
    default: return 0;
  }
}

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_block_size(int bs) { return bs == 16 || bs == 32; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline pa_status launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Shared-prefix (cascade) plan, device arrays: prefix_len[num_seqs],
// groups[ngroups][3] = {first member, member count, prefix tokens},
// members[] = sequence indices; max_prefix = largest prefix, max_members =
// largest group, max_rest = longest context part outside its group's prefix
// (host values).
struct CascadePlan {
  const int32_t* prefix_len;
  const int32_t* groups;
  const int32_t* members;
  int ngroups;
  int max_prefix;
  int max_members;
  int max_rest;
};

// The step's appended K/V ([num_seqs][H_kv][head_dim], device; fp16 / bf16),
// or nulls: position ctx - 1 of every sequence is the token appended this
// step, not yet in the cache.  The decode wave whose range ends at the
// context patches it into its last group from here and stores it in its
// cache slot (the block write fused into the decode); nothing in the same
// launch reads that slot from memory.
struct NewKV {
  const void* k;
  const void* v;
};

// pa_decode with an optional sequence order (a permutation of 0..num_seqs-1,
// device memory; work-groups are issued in that order) and an optional
// cascade plan and, on the fp16 / bf16 path, the step's appended K/V.
pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int num_seqs, int max_context_len,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float scale, int partition_size, void* workspace,
                      size_t workspace_bytes, int dtype, int flags, const int32_t* order,
                      void* stream, const CascadePlan* plan, const NewKV* nkv);

}  // namespace pa
