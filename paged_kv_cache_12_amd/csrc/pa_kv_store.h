// Placement of a new token's K and V in the cache layout, shared by the block
// write (pa_write_kv) and the fused staging + write kernel of the decode step.
//
//   K (block b, head h, token tt, dim i) at tile + ((i / X) * BS + r(tt)) * X + i % X
//   V (block b, head h, token tt, dim i) at tile + ((tt / X) * D + i) * X + tt % X
//
// with tile = (b * H + h) * BS * D, X = 16 / element bytes and r(tt) the row
// of token tt in a K slab (tokens with bit 2 clear first).
#pragma once

#include "pa_internal.h"

namespace pa {

// Stores the 16-byte vector jv (dims jv*X .. jv*X+X-1) of token t, head h of
// k_new / v_new ([tokens][H][D]) at cache slot `slot` (already range-checked).
// E is the element storage type (uint16_t for fp16/bf16, uint32_t for fp32).
template <typename E>
__device__ __forceinline__ void store_token_vec(const E* __restrict__ k_new,
                                                const E* __restrict__ v_new, E* __restrict__ kc,
                                                E* __restrict__ vc, int64_t t, int h, int jv,
                                                int64_t slot, int H, int D, int BS) {
  constexpr int X = 16 / sizeof(E);
  const int64_t b = slot / BS;
  const int tt = static_cast<int>(slot - b * BS);
  const int64_t src = (t * H + h) * D + jv * X;
  const int64_t tile = (b * H + h) * static_cast<int64_t>(BS) * D;
  const int kr = ((tt & 4) ? BS / 2 : 0) + 4 * (tt >> 3) + (tt & 3);
  *reinterpret_cast<u32x4*>(kc + tile + (static_cast<int64_t>(jv) * BS + kr) * X) =
      *reinterpret_cast<const u32x4*>(k_new + src);
  union {
    u32x4 v;
    E e[X];
  } vals;
  vals.v = *reinterpret_cast<const u32x4*>(v_new + src);
  E* vdst = vc + tile + (static_cast<int64_t>(tt / X) * D + jv * X) * X + tt % X;
#pragma unroll
  for (int e = 0; e < X; ++e) vdst[e * X] = vals.e[e];
}

}  // namespace pa
