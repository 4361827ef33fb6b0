// Paged decode attention (pa_decode): the block read fused with attention of
// the vLLM encyclopedia entry (tonho.wtf), sections "como funciona" (scores of
// one block at a time, output accumulated against the same block's values,
// blocks anywhere in memory) and "o que isso custou" (the fused kernel).
//
// Work unit: one wavefront per (partition of the context, KV head, sequence).
// A partition is a run of `part` tokens (whole context when part == 0); its
// result is either the final output (one partition) or a partial (running max
// m in log2 units, sum l, unnormalised output o) merged by decode_reduce.
//
// fp16 / bf16 path (decode_part_mfma): the G query heads that share a KV head
// (GQA) are the N = 16 columns of 16x16x32 MFMAs, so one KV read serves the
// whole group.  Per 32-token group:
//   S^T[token][head] = K[token][:] . Q[head][:]       2 MFMA rows-halves x D/32
//   online softmax on S (per-lane values, two cross-lane max steps)
//   O^T[dim][head] += V^T[dim][token] . P^T[token][head]   D/16 MFMAs
// The QK output layout (lane group g holds tokens 8g..8g+7 of a head column)
// is exactly the PV B-operand layout, so P never leaves its lane.  The cache
// layout makes every K and V operand a 16-byte load straight from HBM in which
// each quad of lanes reads 64 contiguous bytes; no LDS staging is needed.
//
// MFMA 16x16x32 operand layout (lane l, g = l / 16, c = l % 16):
//   A[row c][k 8g..8g+7], B[k 8g..8g+7][col c], D[row 4g+r][col c], r = 0..3.
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x4 mma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<_Float16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x4 mma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

struct Span {
  int ctx, nparts, t0, t1;
};

// Clamped context and this work-group's token range.
__device__ __forceinline__ Span partition_span(const int32_t* ctx_lens, int s, int max_tokens,
                                               int part, int p) {
  Span sp;
  int ctx = ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > max_tokens ? max_tokens : ctx);
  sp.ctx = ctx;
  sp.nparts = part > 0 ? ((ctx + part - 1) / part > 1 ? (ctx + part - 1) / part : 1) : 1;
  sp.t0 = part > 0 ? p * part : 0;
  sp.t1 = part > 0 ? (ctx < sp.t0 + part ? ctx : sp.t0 + part) : ctx;
  return sp;
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(64) void decode_part_mfma(
    T* __restrict__ out, float* __restrict__ ws_o, float2* __restrict__ ws_ml,
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int maxb, const int32_t* __restrict__ ctx_lens,
    int max_tokens, int H_q, int H_kv, int G, int n_hg, int num_blocks, float scale_log2,
    int part, int maxP) {
  typedef Mfma<T> M;
  typedef typename M::v8 v8;
  constexpr int NC = D / 32;    // QK k-chunks of 32 dims
  constexpr int NJ = D / 16;    // PV output chunks of 16 dims
  constexpr int BPT = 32 / BS;  // blocks per 32-token group
  constexpr int TILE = BS * D;  // elements per (block, head) tile

  const int lane = threadIdx.x;
  const int c = lane & 15;  // MFMA row/column index within a lane group
  const int g = lane >> 4;  // lane group
  const int p = blockIdx.x;
  const int kvh = blockIdx.y / n_hg;
  const int hg = blockIdx.y - kvh * n_hg;
  const int s = blockIdx.z;

  const Span sp = partition_span(ctx_lens, s, max_tokens, part, p);
  if (p >= sp.nparts) return;
  const int t0 = sp.t0, t1 = sp.t1;

  const int hin = hg * 16 + c;  // head within the GQA group
  const bool hvalid = hin < G;
  const int qh = kvh * G + hin;

  // B operand of QK: Q[head c][dims 8(4k+g) .. +8] for chunk k.
  v8 qop[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    if (hvalid)
      qop[k] = *reinterpret_cast<const v8*>(q + (static_cast<int64_t>(s) * H_q + qh) * D +
                                            (4 * k + g) * 8);
    else
      qop[k] = v8{};
  }

  f32x4 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int32_t* bt = block_tables + static_cast<int64_t>(s) * maxb;
  const int64_t blk_stride = static_cast<int64_t>(H_kv) * TILE;
  const T* kh = kc + static_cast<int64_t>(kvh) * TILE;
  const T* vh = vc + static_cast<int64_t>(kvh) * TILE;

  // Token (within the 32-token group) whose K row this lane feeds to QK MFMA h:
  // row c holds token 8(c/4) + 4h + c%4, so that output lane group g, register
  // r of MFMA h is token 8g + 4h + r.
  int ku[2], kblk[2], krow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ku[h] = 8 * (c >> 2) + 4 * h + (c & 3);
    kblk[h] = ku[h] / BS;
    krow[h] = ku[h] % BS;
  }
  // V: lane group g feeds tokens 8g .. 8g+7: block vblk, slab vslab.
  const int vblk = (8 * g) / BS;
  const int vslab = ((8 * g) % BS) / 8;

  for (int tg = t0; tg < t1; tg += 32) {
    int pb[BPT];
    const int lb0 = tg / BS;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      int b = -1;
      if ((lb0 + j) * BS < t1) b = bt[lb0 + j];
      if (b < 0 || b >= num_blocks) b = (j == 0) ? 0 : pb[0];
      pb[j] = b;
    }
    v8 kr[2][NC];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const T* base = kh + pb[kblk[h]] * blk_stride + krow[h] * 8;
#pragma unroll
      for (int k = 0; k < NC; ++k)
        kr[h][k] = *reinterpret_cast<const v8*>(base + (4 * k + g) * (BS * 8));
    }
    v8 vr[NJ];
    {
      const T* base = vh + pb[vblk] * blk_stride + vslab * (D * 8) + c * 8;
#pragma unroll
      for (int j = 0; j < NJ; ++j) vr[j] = *reinterpret_cast<const v8*>(base + 16 * j * 8);
    }

    // scores
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NC; ++k) sacc[h] = M::mma(kr[h][k], qop[k], sacc[h]);
    }
    const int rem = t1 - tg;  // valid tokens in this group (>= 1)
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = 8 * g + 4 * h + r;
        x[4 * h + r] = (u < rem) ? sacc[h][r] * scale_log2 : -INFINITY;
      }
    float mloc = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mloc = fmaxf(mloc, x[i]);
    mloc = xor_max(mloc, 16);
    mloc = xor_max(mloc, 32);
    const float mnew = fmaxf(m, mloc);
    const float alpha = fast_exp2(m - mnew);
    float psum = 0.f;
    v8 pop;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = fast_exp2(x[i] - mnew);
      psum += e;
      pop[i] = static_cast<T>(e);
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] *= alpha;

    if (rem < 32) {
      // tail: positions past the context may hold anything (0 * NaN = NaN)
      const int nv = rem - 8 * g;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i >= nv) vr[j][i] = static_cast<T>(0.f);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] = M::mma(vr[j], pop, o[j]);
  }

  float lt = xor_sum(l, 16);
  lt = xor_sum(lt, 32);
  if (!hvalid) return;
  const int64_t row = static_cast<int64_t>(s) * H_q + qh;
  if (sp.nparts == 1) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    T* dst = out + row * D + 4 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[16 * j + r] = static_cast<T>(o[j][r] * inv);
  } else {
    float* dst = ws_o + (row * maxP + p) * D + 4 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j) = o[j];
    if (g == 0) ws_ml[row * maxP + p] = make_float2(m, lt);
  }
}

// fp32 path: one wavefront per (partition, query head, sequence).  QK: lane t
// (< BS) owns token t of the block; PV: lane owns dims lane and lane + 64.
template <int D, int BS>
__global__ __launch_bounds__(64) void decode_part_f32(
    float* __restrict__ out, float* __restrict__ ws_o, float2* __restrict__ ws_ml,
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int maxb, const int32_t* __restrict__ ctx_lens,
    int max_tokens, int H_q, int H_kv, int G, int num_blocks, float scale_log2, int part,
    int maxP) {
  constexpr int X = 4;
  constexpr int DPL = D / 64;
  constexpr int TILE = BS * D;
  const int lane = threadIdx.x;
  const int p = blockIdx.x;
  const int qh = blockIdx.y;
  const int s = blockIdx.z;
  const int kvh = qh / G;

  const Span sp = partition_span(ctx_lens, s, max_tokens, part, p);
  if (p >= sp.nparts) return;
  const int t0 = sp.t0, t1 = sp.t1;

  __shared__ float qs[D];
  const int64_t row = static_cast<int64_t>(s) * H_q + qh;
  for (int i = lane; i < D; i += 64) qs[i] = q[row * D + i];
  __syncthreads();

  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int32_t* bt = block_tables + static_cast<int64_t>(s) * maxb;

  for (int lb = t0 / BS; lb * BS < t1; ++lb) {
    int b = bt[lb];
    if (b < 0 || b >= num_blocks) b = 0;
    const float* kt = kc + (static_cast<int64_t>(b) * H_kv + kvh) * TILE;
    const float* vt = vc + (static_cast<int64_t>(b) * H_kv + kvh) * TILE;
    const int nval = (t1 - lb * BS) < BS ? (t1 - lb * BS) : BS;
    float sc = -INFINITY;
    if (lane < BS) {
      float dot = 0.f;
#pragma unroll 4
      for (int j = 0; j < D / X; ++j) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(kt + (j * BS + lane) * X);
        dot = fmaf(qs[4 * j + 0], kv[0], dot);
        dot = fmaf(qs[4 * j + 1], kv[1], dot);
        dot = fmaf(qs[4 * j + 2], kv[2], dot);
        dot = fmaf(qs[4 * j + 3], kv[3], dot);
      }
      if (lane < nval) sc = dot * scale_log2;
    }
    float bm = sc;
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) bm = xor_max(bm, mask);
    const float mnew = fmaxf(m, bm);
    const float alpha = fast_exp2(m - mnew);
    const float pe = (lane < nval) ? fast_exp2(sc - mnew) : 0.f;
    float ps = pe;
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) ps = xor_sum(ps, mask);
    l = l * alpha + ps;
    m = mnew;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] *= alpha;
#pragma unroll
    for (int t4 = 0; t4 < BS / X; ++t4) {
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const f32x4 vv =
            *reinterpret_cast<const f32x4*>(vt + (t4 * D + lane + 64 * k) * X);
#pragma unroll
        for (int e = 0; e < X; ++e) {
          const int t = t4 * X + e;
          const float pt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), t));
          if (t < nval) acc[k] = fmaf(pt, vv[e], acc[k]);
        }
      }
    }
  }
  if (sp.nparts == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[row * D + lane + 64 * k] = acc[k] * inv;
  } else {
    float* dst = ws_o + (row * maxP + p) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) dst[lane + 64 * k] = acc[k];
    if (lane == 0) ws_ml[row * maxP + p] = make_float2(m, l);
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
// M = max m_p, L = sum 2^(m_p - M) l_p, out = sum 2^(m_p - M) o_p / L, in
// ascending p.  One thread per output dim.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_reduce(T* __restrict__ out,
                                                   const float* __restrict__ ws_o,
                                                   const float2* __restrict__ ws_ml,
                                                   const int32_t* __restrict__ ctx_lens,
                                                   int max_tokens, int H_q, int part, int maxP) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const Span sp = partition_span(ctx_lens, s, max_tokens, part, 0);
  if (sp.nparts <= 1) return;
  const int np = sp.nparts < maxP ? sp.nparts : maxP;
  const int64_t row = static_cast<int64_t>(s) * H_q + h;
  const float2* ml = ws_ml + row * maxP;
  const float* o = ws_o + row * maxP * D + d;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[p].x);
  float L = 0.f, acc = 0.f;
  for (int p = 0; p < np; ++p) {
    const float2 v = ml[p];
    const float w = fast_exp2(v.x - M);
    L = fmaf(w, v.y, L);
    acc = fmaf(w, o[static_cast<int64_t>(p) * D], acc);
  }
  out[row * D + d] = static_cast<T>(acc / L);
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  int maxb;
  const int32_t* lens;
  int B, max_tokens, H_q, H_kv, G, num_blocks;
  float scale_log2;
  int part, maxP;
  float* ws_o;
  float2* ws_ml;
  hipStream_t st;
};

template <typename T, int D, int BS>
void launch_mfma(const DecodeArgs& a) {
  const int n_hg = (a.G + 15) / 16;
  hipLaunchKernelGGL((decode_part_mfma<T, D, BS>), dim3(a.maxP, a.H_kv * n_hg, a.B), dim3(64), 0,
                     a.st, static_cast<T*>(a.out), a.ws_o, a.ws_ml, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.kc), static_cast<const T*>(a.vc), a.bt, a.maxb,
                     a.lens, a.max_tokens, a.H_q, a.H_kv, a.G, n_hg, a.num_blocks, a.scale_log2,
                     a.part, a.maxP);
  if (a.maxP > 1)
    hipLaunchKernelGGL((decode_reduce<T, D>), dim3(a.H_q, a.B), dim3(D), 0, a.st,
                       static_cast<T*>(a.out), a.ws_o, a.ws_ml, a.lens, a.max_tokens, a.H_q,
                       a.part, a.maxP);
}

template <int D, int BS>
void launch_f32(const DecodeArgs& a) {
  hipLaunchKernelGGL((decode_part_f32<D, BS>), dim3(a.maxP, a.H_q, a.B), dim3(64), 0, a.st,
                     static_cast<float*>(a.out), a.ws_o, a.ws_ml, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.kc), static_cast<const float*>(a.vc), a.bt,
                     a.maxb, a.lens, a.max_tokens, a.H_q, a.H_kv, a.G, a.num_blocks,
                     a.scale_log2, a.part, a.maxP);
  if (a.maxP > 1)
    hipLaunchKernelGGL((decode_reduce<float, D>), dim3(a.H_q, a.B), dim3(D), 0, a.st,
                       static_cast<float*>(a.out), a.ws_o, a.ws_ml, a.lens, a.max_tokens, a.H_q,
                       a.part, a.maxP);
}

template <typename T>
void dispatch_mfma(const DecodeArgs& a, int D, int BS) {
  if (D == 64 && BS == 16) launch_mfma<T, 64, 16>(a);
  else if (D == 64 && BS == 32) launch_mfma<T, 64, 32>(a);
  else if (D == 128 && BS == 16) launch_mfma<T, 128, 16>(a);
  else launch_mfma<T, 128, 32>(a);
}

inline int num_partitions(int max_ctx, int part) {
  if (part <= 0 || max_ctx <= part) return 1;
  return (max_ctx + part - 1) / part;
}

}  // namespace pa

using namespace pa;

PA_EXPORT size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                          int max_context_len, int partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  const int maxP = num_partitions(max_context_len, partition_size);
  if (maxP <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * maxP;
  const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return o_bytes + rows * sizeof(float2);
}

PA_EXPORT pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int num_seqs, int max_context_len,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, float scale, int partition_size, void* workspace,
                              size_t workspace_bytes, int dtype, void* stream) {
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_context_len < 0 || max_blocks_per_seq < 0 || partition_size < 0)
    return PA_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (partition_size % 32 != 0) return PA_ERR_INVALID;
  if (!std::isfinite(scale)) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_context_len) >
      static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID;
  if (num_seqs > 65535 || static_cast<int64_t>(num_kv_heads) * 16 > 65535) return PA_ERR_INVALID;
  const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                               partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_INVALID;

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.bt = block_tables;
  a.maxb = max_blocks_per_seq;
  a.lens = context_lens;
  a.B = num_seqs;
  a.max_tokens = max_context_len;
  a.H_q = num_q_heads;
  a.H_kv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.num_blocks = num_blocks;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.maxP = num_partitions(max_context_len, partition_size);
  a.part = a.maxP > 1 ? partition_size : 0;
  if (need > 0) {
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * a.maxP;
    const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + o_bytes);
  } else {
    a.ws_o = nullptr;
    a.ws_ml = nullptr;
  }
  a.st = static_cast<hipStream_t>(stream);

  switch (dtype) {
    case PA_BF16: dispatch_mfma<__bf16>(a, head_dim, block_size); break;
    case PA_F16: dispatch_mfma<_Float16>(a, head_dim, block_size); break;
    default:
      if (head_dim == 64 && block_size == 16) launch_f32<64, 16>(a);
      else if (head_dim == 64 && block_size == 32) launch_f32<64, 32>(a);
      else if (head_dim == 128 && block_size == 16) launch_f32<128, 16>(a);
      else launch_f32<128, 32>(a);
      break;
  }
  return launch_status();
}
