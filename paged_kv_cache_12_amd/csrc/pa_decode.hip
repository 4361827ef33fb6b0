// Paged decode attention (pa_decode): the block read fused with attention of
// the vLLM encyclopedia entry (tonho.wtf), sections "como funciona" (scores of
// one block at a time, output accumulated against the same block's values,
// blocks anywhere in memory) and "o que isso custou" (the fused kernel).
//
// Work unit: a work-group of NW wavefronts per (chunk of NW partitions, KV
// head [x head group], sequence).  Each wave runs one partition, a run of
// `part` tokens (a range that fits one chunk, always the case when part == 0,
// is instead split evenly over the waves) with its own running state (max m
// in log2 units, sum l, unnormalised output o); the waves merge in LDS and
// the work-group writes the final output, or one partial per chunk that
// decode_reduce merges.  With an appended token (the decode step), the wave
// that ends each context also performs its block write.  The shared-prefix
// (cascade) modes are described at decode_part_mfma's modes below.
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
#include <algorithm>
#include <climits>
#include <mutex>

#include "pa_kv_store.h"


namespace pa {

// Tokens a work-group of the fp16/bf16 path aims to cover: NW partitions of
// `part` tokens with NW = kChunkTokens / part (1..8), 8 waves when unsplit.
constexpr int kChunkTokens = 2048;

// Plain decode of contexts of at least this many partitions runs 6 waves per
// work-group where the rule above gives 4: a third fewer partial writes in
// the read stream, and two work-groups still fill a CU's 12 wave slots
// (8 waves would leave 4 idle).  Measured on 32k-131k contexts with
// 512-token partitions: 477 -> 457 us; shorter ranges lose more to idle waves
// in a sequence's last chunk than they gain.
constexpr int kLongParts = 64;

// Waves per SIMD the one-tile kernels are compiled for (at most 168 VGPRs);
// the two-tile prefix pass needs more registers and runs two.
constexpr int kWavesPerSimd = 3;

// Scores more than this many log2 units above the running reference trigger a
// rescale; weights fed to the PV product are at most 2^kRescaleLog2.
constexpr float kRescaleLog2 = 8.0f;

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

struct ChunkSpan {
  int nchunks, t0, t1;
};

// Chunks of nw partitions covering n tokens (at least one, also for n == 0).
__device__ __forceinline__ int chunks_n(int n, int part, int nw) {
  if (part <= 0) return 1;
  const int nparts = (n + part - 1) / part;
  return nparts > nw ? (nparts + nw - 1) / nw : 1;
}
template <int NW>
__device__ __forceinline__ int chunks_of(int n, int part) {
  return chunks_n(n, part, NW);
}

// Tokens of a shared prefix of length L that the prefix pass covers, for a
// context of ctx tokens: L clamped to [0, ctx] and rounded down to whole
// 32-token groups, so that the prefix pass and the rest both run on group
// boundaries (a plan's L need not be a multiple of 32; the tokens cut off
// move to the rest, and the result is the same attention).
__device__ __forceinline__ int prefix_tokens(int L, int ctx) {
  return (L < 0 ? 0 : (L > ctx ? ctx : L)) & ~31;
}

// Token range of wave `wave` in chunk `ch` over tokens [lo, hi): partition
// ch * NW + wave of `part` tokens; a range that fits one chunk (always with
// part == 0) is split evenly into NW runs of whole 32-token groups, so that
// no wave of the work-group idles.
template <int NW>
__device__ __forceinline__ ChunkSpan range_span(int lo, int hi, int part, int ch, int wave) {
  ChunkSpan sp;
  const int n = hi > lo ? hi - lo : 0;
  sp.nchunks = chunks_of<NW>(n, part);
  const int unit = sp.nchunks > 1 ? part : (((n + NW - 1) / NW) + 31) & ~31;
  const int64_t a = (static_cast<int64_t>(ch) * NW + wave) * unit;
  sp.t0 = lo + (a < n ? static_cast<int>(a) : n);
  sp.t1 = lo + (a + unit < n ? static_cast<int>(a + unit) : n);
  return sp;
}

// Grid linearisation.  Streaming (no aliased blocks): chunk fastest, then
// head, then sequence.  Aliased blocks: work-groups are dealt to the 8 XCDs
// round-robin by linear id, so with (KV head x head group) count HG a multiple
// of 8 the id is split as id = 8 j + x: XCD x serves heads x, x+8, ...; along
// j the head varies fastest, then the sequence, then the chunk, and sequences
// that alias the same blocks (shared prefixes, parallel samples) read them one
// after the other from the same XCD's L2.
struct WorkItem {
  int chunk, hgl, seq;
};

template <bool ALIASED>
__device__ __forceinline__ WorkItem work_item(int id, int HG, int B, int maxC) {
  WorkItem w;
  if (!ALIASED || (HG & 7) != 0) {
    w.chunk = id % maxC;
    const int rest = id / maxC;
    w.hgl = rest % HG;
    w.seq = rest / HG;
    return w;
  }
  const int x = id & 7, j = id >> 3, sub = HG >> 3;
  w.hgl = x + 8 * (j % sub);
  const int rest = j / sub;
  w.seq = rest % B;
  w.chunk = rest / B;
  return w;
}

// Registers holding one 32-token group's operands.
template <typename T, int D>
struct GroupTiles {
  typedef typename Mfma<T>::v8 v8;
  v8 k[2][D / 32];
  v8 v[D / 16];
};

// K/V tile loads: non-temporal when every block is read once per step (NT),
// ordinary cached loads when blocks are aliased by several sequences.
template <typename V, bool NT>
__device__ __forceinline__ V load16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  return *reinterpret_cast<const V*>(p);
}

// Row of token t inside a K slab (tokens with bit 2 clear first).
template <int BS>
__device__ __forceinline__ int k_row(int t) {
  return ((t & 4) ? BS / 2 : 0) + 4 * (t >> 3) + (t & 3);
}

// Block-table window: lane i holds entry lb_base + i of the sequence's table
// (64 entries per window, refilled when a group crosses it).  Entries past the
// context, or out of range, read as block 0; the tokens they stand for are
// masked, so the value only has to be a valid block.
struct TableWindow {
  int lb_base;
  int ids;  // this lane's entry
};

__device__ __forceinline__ void fill_window(TableWindow& w, const int32_t* __restrict__ bt,
                                            int lb_base, int nb_valid, int num_blocks,
                                            int lane) {
  w.lb_base = lb_base;
  int b = 0;
  if (lb_base + lane < nb_valid) b = bt[lb_base + lane];
  if (b < 0 || b >= num_blocks) b = 0;
  w.ids = b;
}

template <typename T, int D, int BS, bool NT>
__device__ __forceinline__ void load_group(GroupTiles<T, D>& G, TableWindow& w,
                                           const int32_t* __restrict__ bt, int tg, int nb_valid,
                                           int num_blocks, const T* kh, const T* vh,
                                           int64_t blk_stride, const int* kblk, const int* krow,
                                           int vblk, int vslab, int g, int c, int lane) {
  typedef typename Mfma<T>::v8 v8;
  constexpr int NC = D / 32, NJ = D / 16, BPT = 32 / BS;
  const int lb0 = tg / BS;
  if (lb0 + BPT - 1 >= w.lb_base + 64) fill_window(w, bt, lb0, nb_valid, num_blocks, lane);
  // block offsets are wave-uniform (scalar multiplies); each lane then only
  // selects the one of its block
  int64_t boff[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    boff[j] = static_cast<int64_t>(__builtin_amdgcn_readlane(w.ids, lb0 + j - w.lb_base)) *
              blk_stride;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const T* base = kh + boff[kblk[h]] + krow[h] * 8;
#pragma unroll
    for (int k = 0; k < NC; ++k)
      G.k[h][k] = load16<v8, NT>(base + (4 * k + g) * (BS * 8));
  }
  const T* base = vh + boff[vblk] + vslab * (D * 8) + c * 8;
#pragma unroll
  for (int j = 0; j < NJ; ++j) G.v[j] = load16<v8, NT>(base + 16 * j * 8);
}

// QK and the online-softmax update for one 32-token group; returns the
// weights as the PV B operand.  TAIL: only the first `rem` tokens of the group
// are inside the context (the last group of a range); the others are masked
// out of the scores.
template <typename T, int D, bool TAIL>
__device__ __forceinline__ typename Mfma<T>::v8 qk_softmax(const GroupTiles<T, D>& G,
                                                           const typename Mfma<T>::v8* qop,
                                                           f32x4* o, float& m, float& l, int rem,
                                                           int g, float scale_log2) {
  typedef Mfma<T> M;
  typedef typename M::v8 v8;
  constexpr int NC = D / 32, NJ = D / 16;
  f32x4 sacc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NC; ++k) sacc[h] = M::mma(G.k[h][k], qop[k], sacc[h]);
  }
  // raw scores of tokens 8g + 4h + r (scale > 0, so the max commutes with it)
  float x[8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[4 * h + r] = sacc[h][r];
      if (TAIL && 8 * g + 4 * h + r >= rem) x[4 * h + r] = -INFINITY;
    }
  float mraw = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  const float mloc = mraw * scale_log2;
  // Lazy rescale: the reference m only moves when a score exceeds it by more
  // than kRescaleLog2, so weights stay <= 2^kRescaleLog2 and the accumulators
  // are rescaled only on this wave-uniform, rarely taken path.
  if (__builtin_amdgcn_ballot_w64(mloc > m + kRescaleLog2)) {
    __asm__ volatile("");  // keep the path a real branch (not speculated)
    float mw = xor_max(mloc, 16);
    mw = xor_max(mw, 32);
    const float mnew = fmaxf(m, mw);
    const float alpha = fast_exp2(m - mnew);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] *= alpha;
    m = mnew;
  }
  float psum = 0.f;
  v8 pop;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float e = fast_exp2(fmaf(x[i], scale_log2, -m));
    psum += e;
    pop[i] = static_cast<T>(e);
  }
  l += psum;
  return pop;
}

// PV for one 32-token group.  TAIL: V lanes of tokens past `rem` are zeroed
// first, since slots past the fill may hold anything (0 * NaN = NaN).
template <typename T, int D, bool TAIL>
__device__ __forceinline__ void pv(GroupTiles<T, D>& G, typename Mfma<T>::v8 pop, f32x4* o,
                                   int rem, int g) {
  typedef Mfma<T> M;
  typedef typename M::v8 v8;
  constexpr int NJ = D / 16;
  if (TAIL) {
    // keep the first nv of this lane's 8 V elements (16-bit lanes of 4 dwords)
    const int nv = rem - 8 * g;
    u32x4 keep;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      keep[w] = (2 * w < nv ? 0x0000FFFFu : 0u) | (2 * w + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 bits = __builtin_bit_cast(u32x4, G.v[j]);
      bits &= keep;
      G.v[j] = __builtin_bit_cast(v8, bits);
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = M::mma(G.v[j], pop, o[j]);
}

// Replaces token u (0..31) of a loaded group by the appended token's K row
// and V column (k_row / v_col: its D values): the K rows of MFMA half h hold
// token 8(c/4) + 4h + c%4 in lane c, and V lane group g holds tokens
// 8g .. 8g+7 of dims 16j + c.
template <typename T, int D>
__device__ __forceinline__ void patch_new_token(GroupTiles<T, D>& G, const T* k_row,
                                                const T* v_col, int u, int g, int c) {
  typedef typename Mfma<T>::v8 v8;
  constexpr int NC = D / 32, NJ = D / 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (8 * (c >> 2) + 4 * h + (c & 3) == u) {
#pragma unroll
      for (int k = 0; k < NC; ++k)
        G.k[h][k] = *reinterpret_cast<const v8*>(k_row + (4 * k + g) * 8);
    }
  }
  if ((u >> 3) == g) {
    // element u % 8 of each V vector: 16-bit half (u & 1) of dword (u & 7) / 2
    // (selects over constant indices keep the vectors in registers)
    const int w = (u & 7) >> 1;
    const bool hi_half = u & 1;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t val = __builtin_bit_cast(uint16_t, v_col[16 * j + c]);
      u32x4 bits = __builtin_bit_cast(u32x4, G.v[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t put = hi_half ? ((bits[i] & 0x0000FFFFu) | (val << 16))
                                     : ((bits[i] & 0xFFFF0000u) | val);
        bits[i] = i == w ? put : bits[i];
      }
      G.v[j] = __builtin_bit_cast(v8, bits);
    }
  }
}

// QK, online-softmax update and PV for one 32-token group.
template <typename T, int D, bool TAIL>
__device__ __forceinline__ void compute_group(GroupTiles<T, D>& G,
                                              const typename Mfma<T>::v8* qop, f32x4* o,
                                              float& m, float& l, int rem, int g,
                                              float scale_log2) {
  const typename Mfma<T>::v8 pop = qk_softmax<T, D, TAIL>(G, qop, o, m, l, rem, g, scale_log2);
  pv<T, D, TAIL>(G, pop, o, rem, g);
}

// Work decomposition of decode_part_mfma:
//   kPlain   one work-group per (chunk, KV head [x head group], sequence);
//   kSuffix  the same over tokens [prefix_len[s], ctx) of each sequence, always
//            writing partials after the sequence's prefix-pass partials when
//            prefix_len[s] > 0;
//   kPrefix  one work-group per (chunk, KV head, column group): the sequences
//            of a group share the physical blocks of their first L tokens, and
//            their queries fill the 16 MFMA columns (member c / G, head c % G),
//            so each K/V load serves all of them; partials only;
//   kPrefix2 the same with two 16-column tiles per K/V load (groups of up to
//            32 / G sequences).
enum { kPlain = 0, kSuffix = 1, kPrefix = 2, kPrefix2 = 3 };

// The one-tile prefix pass runs at most kPrefixWaves waves per work-group
// (three work-groups fill a CU's wave slots); the two-tile form, two waves
// per SIMD, runs twice as many (up to 8: one work-group per CU), so that a
// 4096-token prefix with 512-token partitions is one chunk and leaves one
// partial per row, half the partial bytes the suffix pass then reads.  The
// prefix pass's wave count travels in Cascade::prefix_nw, with which the
// suffix pass and the reduce count a row's prefix chunks.
constexpr int kPrefixWaves = 4;
template <int NW>
struct PrefixNW {
  static constexpr int value = NW > kPrefixWaves ? kPrefixWaves : NW;
};
template <int NW>
struct Prefix2NW {
  static constexpr int value = 2 * PrefixNW<NW>::value > 8 ? 8 : 2 * PrefixNW<NW>::value;
};

// Cascade description on the device: prefix_len[B]; groups[ng][3] =
// {first member, member count, L}; members[] = sequence indices; prefix_nw:
// waves per work-group of the prefix pass that ran.
struct Cascade {
  const int32_t* prefix_len;
  const int32_t* groups;
  const int32_t* members;
  int ngroups;
  int prefix_nw;
};

template <typename T, int D, int BS, int NW, bool NT, int MODE>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(MODE == kPrefix2 ? 2 : kWavesPerSimd)))
void decode_part_mfma(
    T* __restrict__ out, float* __restrict__ ws_o, float2* __restrict__ ws_ml,
    const T* __restrict__ q, const T* kc, const T* vc,
    const int32_t* __restrict__ block_tables, int maxb, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ order, int B, int max_tokens, int H_q, int H_kv, int G,
    int n_hg, int num_blocks, float scale_log2, int part, int maxC, int ws_stride, Cascade cas,
    NewKV nkv) {
  typedef Mfma<T> M;
  typedef typename M::v8 v8;
  constexpr int NC = D / 32;    // QK k-chunks of 32 dims
  constexpr int NJ = D / 16;    // PV output chunks of 16 dims
  constexpr int TILE = BS * D;  // elements per (block, head) tile

  // the wave index through readfirstlane: the compiler then keeps every
  // per-wave value (token range, loop counter, block offsets) in scalar
  // registers and runs the loop on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;  // MFMA row/column index within a lane group
  const int g = lane >> 4;  // lane group
  const WorkItem wi =
      work_item<!NT>(blockIdx.x, H_kv * n_hg, MODE >= kPrefix ? cas.ngroups : B, maxC);
  const int ch = wi.chunk;
  const int kvh = wi.hgl / n_hg;
  const int hg = wi.hgl - kvh * n_hg;

  // the sequence whose table is read, each tile column's sequence and head,
  // and the partial slot of chunk 0; the prefix pass runs TT column tiles
  // (TT x 16 columns) on every loaded K/V group
  constexpr bool PREFIX = MODE == kPrefix || MODE == kPrefix2;
  constexpr int TT = MODE == kPrefix2 ? 2 : 1;
  int s, slot0 = 0, lo = 0, hi;
  int s_col[TT], hin[TT];
  bool hvalid[TT];
  if constexpr (PREFIX) {
    const int gi = wi.seq;
    const int first = cas.groups[3 * gi], count = cas.groups[3 * gi + 1];
    hi = prefix_tokens(cas.groups[3 * gi + 2], INT_MAX);
    s = cas.members[first];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int col = 16 * t + c;
      const int mi = col / G;
      hin[t] = col - mi * G;
      hvalid[t] = mi < count;
      s_col[t] = hvalid[t] ? cas.members[first + mi] : s;
    }
  } else {
    s = order ? order[wi.seq] : wi.seq;
    if (s < 0 || s >= B) return;
    int ctx = ctx_lens[s];
    hi = ctx < 0 ? 0 : (ctx > max_tokens ? max_tokens : ctx);
    if constexpr (MODE == kSuffix) {
      lo = prefix_tokens(cas.prefix_len[s], hi);
      if (lo > 0) slot0 = chunks_n(lo, part, cas.prefix_nw);
    }
    hin[0] = hg * 16 + c;  // head within the GQA group
    hvalid[0] = hin[0] < G;
    s_col[0] = s;
  }
  const ChunkSpan sp = range_span<NW>(lo, hi, part, ch, wave);
  if (ch >= sp.nchunks) return;  // uniform over the work-group
  const int t0 = sp.t0, t1 = sp.t1;
  // the final output is written here for a context in one chunk; a suffix in
  // one chunk first merges the prefix pass's partials of its rows
  const bool final_out = !PREFIX && sp.nchunks == 1;

  // B operand of QK: Q[column c][dims 8(4k+g) .. +8] for chunk k.
  v8 qop[TT][NC];
  f32x4 o[TT][NJ];
  float m[TT], l[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int qh = kvh * G + hin[t];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      if (hvalid[t])
        qop[t][k] = *reinterpret_cast<const v8*>(
            q + (static_cast<int64_t>(s_col[t]) * H_q + qh) * D + (4 * k + g) * 8);
      else
        qop[t][k] = v8{};
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    l[t] = 0.f;
  }

  const int32_t* bt = block_tables + static_cast<int64_t>(s) * maxb;
  const int64_t blk_stride = static_cast<int64_t>(H_kv) * TILE;
  const T* kh = kc + static_cast<int64_t>(kvh) * TILE;
  const T* vh = vc + static_cast<int64_t>(kvh) * TILE;

  // Token (within the 32-token group) whose K row this lane feeds to QK MFMA h:
  // row c holds token 8(c/4) + 4h + c%4, so that output lane group g, register
  // r of MFMA h is token 8g + 4h + r.
  int kblk[2], krow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = 8 * (c >> 2) + 4 * h + (c & 3);
    kblk[h] = u / BS;
    krow[h] = k_row<BS>(u % BS);
  }
  // V: lane group g feeds tokens 8g .. 8g+7: block vblk, slab vslab.
  const int vblk = (8 * g) / BS;
  const int vslab = ((8 * g) % BS) / 8;

  // Full 32-token groups, then at most one partial group at the end; with an
  // appended token, the group holding it is always that last one.
  const bool has_new = !PREFIX && nkv.k != nullptr && t0 < t1 && t1 == hi;
  const int tfull = t0 + ((t1 - t0 - (has_new ? 1 : 0)) & ~31);
  const int nb_valid = (t1 + BS - 1) / BS;  // table entries inside the context
  TableWindow win;
  fill_window(win, bt, t0 / BS, nb_valid, num_blocks, lane);
  int tg = t0;
  if constexpr (D == 64) {
    // head dim 64: a group's K/V is half as many bytes, so two groups are
    // requested per iteration (a wave then has as many bytes in flight as
    // with head dim 128); they are computed in order, as one at a time
    for (; tg + 32 < tfull; tg += 64) {
      GroupTiles<T, D> A, B2;
      load_group<T, D, BS, NT>(A, win, bt, tg, nb_valid, num_blocks, kh, vh, blk_stride, kblk,
                               krow, vblk, vslab, g, c, lane);
      load_group<T, D, BS, NT>(B2, win, bt, tg + 32, nb_valid, num_blocks, kh, vh, blk_stride,
                               kblk, krow, vblk, vslab, g, c, lane);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        compute_group<T, D, false>(A, qop[t], o[t], m[t], l[t], 32, g, scale_log2);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        compute_group<T, D, false>(B2, qop[t], o[t], m[t], l[t], 32, g, scale_log2);
    }
  }
  for (; tg < tfull; tg += 32) {
    GroupTiles<T, D> A;
    load_group<T, D, BS, NT>(A, win, bt, tg, nb_valid, num_blocks, kh, vh, blk_stride, kblk, krow,
                         vblk, vslab, g, c, lane);
#pragma unroll
    for (int t = 0; t < TT; ++t)
      compute_group<T, D, false>(A, qop[t], o[t], m[t], l[t], 32, g, scale_log2);
  }
  if (tg < t1) {
    GroupTiles<T, D> A;
    load_group<T, D, BS, NT>(A, win, bt, tg, nb_valid, num_blocks, kh, vh, blk_stride, kblk, krow,
                         vblk, vslab, g, c, lane);
    if (has_new) {
      const int64_t src = (static_cast<int64_t>(s) * H_kv + kvh) * D;
      patch_new_token<T, D>(A, static_cast<const T*>(nkv.k) + src,
                            static_cast<const T*>(nkv.v) + src, hi - 1 - tg, g, c);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
      compute_group<T, D, true>(A, qop[t], o[t], m[t], l[t], t1 - tg, g, scale_log2);
    if (has_new && lane < D * static_cast<int>(sizeof(T)) / 16) {
      // the block write of the appended token (lane = 16-byte vector)
      const int lb = (hi - 1) / BS;
      const int32_t b = bt[lb];
      if (b >= 0 && b < num_blocks)
        store_token_vec<uint16_t>(static_cast<const uint16_t*>(nkv.k),
                                  static_cast<const uint16_t*>(nkv.v),
                                  reinterpret_cast<uint16_t*>(const_cast<T*>(kc)),
                                  reinterpret_cast<uint16_t*>(const_cast<T*>(vc)), s, kvh, lane,
                                  static_cast<int64_t>(b) * BS + (hi - 1) % BS, H_kv, D, BS);
    }
  }

  float lt[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    lt[t] = xor_sum(l[t], 16);
    lt[t] = xor_sum(lt[t], 32);
  }

  if constexpr (PREFIX && NW > 4) {
    // One merge round: every wave's (m, l, o) goes to LDS; after one barrier
    // each wave combines the NW states for its share of the (tile, 16-dim
    // chunk) slices with weights 2^(m_w - M) and writes those slices of the
    // rows' partials itself (non-temporal: read once by a later launch).
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    __shared__ float all_m[NW][TT][16];
    __shared__ float all_l[NW][TT][16];
    __shared__ f32x4 all_o[NW][TT][NJ][64];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (g == 0) {
        all_m[wave][t][c] = m[t];
        all_l[wave][t][c] = lt[t];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) all_o[wave][t][j][lane] = o[t][j];
    }
    __syncthreads();
    for (int pi = wave; pi < TT * NJ; pi += NW) {  // uniform over the wave
      const int t = pi / NJ, j = pi - t * NJ;
      float mw[NW];
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mw[w] = all_m[w][t][c];
        mm = fmaxf(mm, mw[w]);
      }
      float ls = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - mm);
        ls = fmaf(f, all_l[w][t][c], ls);
        acc += f * all_o[w][t][j][lane];
      }
      bool valid = false;
      int64_t row = 0;
#pragma unroll
      for (int u = 0; u < TT; ++u)
        if (u == t) {
          valid = hvalid[u];
          row = static_cast<int64_t>(s_col[u]) * H_q + kvh * G + hin[u];
        }
      if (!valid) continue;
      const int64_t slot = row * ws_stride + slot0 + ch;
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(ws_o + slot * D + 16 * j + 4 * g));
      if (j == 0 && g == 0)
        __builtin_nontemporal_store(f32x2{mm, ls}, reinterpret_cast<f32x2*>(ws_ml + slot));
    }
    return;
  } else if constexpr (NW > 1) {
    // Merge the waves' states: M = max m_w, weights 2^(m_w - M).
    __shared__ float sh_m[NW][TT][16];
    __shared__ float sh_l[NW][TT][16];
    __shared__ f32x4 sh_o[NW - 1][TT][NJ][64];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (g == 0) {
        sh_m[wave][t][c] = m[t];
        sh_l[wave][t][c] = lt[t];
      }
      if (wave > 0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) sh_o[wave - 1][t][j][lane] = o[t][j];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float mw[NW];
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mw[w] = sh_m[w][t][c];
        mm = fmaxf(mm, mw[w]);
      }
      float f[NW];
      float ls = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        f[w] = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - mm);
        ls = fmaf(f[w], sh_l[w][t][c], ls);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x4 acc = f[0] * o[t][j];
#pragma unroll
        for (int w = 1; w < NW; ++w) acc += f[w] * sh_o[w - 1][t][j][lane];
        o[t][j] = acc;
      }
      m[t] = mm;
      lt[t] = ls;
    }
  }

#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (!hvalid[t]) continue;
    const int64_t row = static_cast<int64_t>(s_col[t]) * H_q + kvh * G + hin[t];
    if constexpr (MODE == kSuffix) {
      if (final_out && slot0 > 0) {
        // M = max over the prefix partials and this state, weights 2^(m_p - M);
        // the reads are issued in batches (8 maxima, then two partials at a
        // time) so that their latencies overlap
        const int64_t base = row * ws_stride;
        float mm = m[t];
        for (int p0 = 0; p0 < slot0; p0 += 8) {
          float mx[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) mx[u] = p0 + u < slot0 ? ws_ml[base + p0 + u].x : -INFINITY;
#pragma unroll
          for (int u = 0; u < 8; ++u) mm = fmaxf(mm, mx[u]);
        }
        const float fs = m[t] == -INFINITY ? 0.f : fast_exp2(m[t] - mm);
        lt[t] *= fs;
#pragma unroll
        for (int j = 0; j < NJ; ++j) o[t][j] *= fs;
        for (int p0 = 0; p0 < slot0; p0 += 2) {
          float2 v[2];
          f32x4 po[2][NJ];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int p = p0 + u < slot0 ? p0 + u : p0;
            v[u] = ws_ml[base + p];
            const float* src = ws_o + (base + p) * D + 4 * g;
#pragma unroll
            for (int j = 0; j < NJ; ++j) po[u][j] = *reinterpret_cast<const f32x4*>(src + 16 * j);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float f =
                p0 + u >= slot0 || v[u].x == -INFINITY ? 0.f : fast_exp2(v[u].x - mm);
            lt[t] = fmaf(f, v[u].y, lt[t]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) o[t][j] += f * po[u][j];
          }
        }
      }
    }
    if (final_out) {
      const float inv = lt[t] > 0.f ? 1.f / lt[t] : 0.f;
      T* dst = out + row * D + 4 * g;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[16 * j + r] = static_cast<T>(o[t][j][r] * inv);
    } else {
      // partials are read once, by a later launch: non-temporal stores keep
      // them from displacing K/V lines in the caches (long context 457 ->
      // 450 us, shared prefix -1.5 us; non-temporal stores of the final
      // outputs measured slightly slower and are not used)
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const int64_t slot = row * ws_stride + slot0 + ch;
      float* dst = ws_o + slot * D + 4 * g;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        __builtin_nontemporal_store(o[t][j], reinterpret_cast<f32x4*>(dst + 16 * j));
      if (g == 0)
        __builtin_nontemporal_store(f32x2{m[t], lt[t]}, reinterpret_cast<f32x2*>(ws_ml + slot));
    }
  }
}

// fp32 path: one wavefront per (partition, query head, sequence).  QK: the
// TPL = 64 / BS lanes of token t (lanes t*TPL ..) each take D / TPL of its
// dims and add their dot products by shuffles; PV: lane owns dims lane and
// lane + 64.  The block table comes in 64-entry windows (one entry per lane),
// and (F32Tile::PREFETCH) the next block's K and V are requested before this
// block's arithmetic, so that the loop does not wait a memory round trip per
// block.
template <int D, int BS>
struct F32Tile {
  static constexpr int X = 4;              // fp32 elements per 16-byte vector
  static constexpr int TPL = 64 / BS;      // QK lanes per token
  static constexpr int NK = D / TPL / X;   // K vectors per lane
  static constexpr int DPL = D / 64;       // PV dims per lane
  static constexpr int NV = BS / X * DPL;  // V vectors per lane
  // the next tile is requested ahead when two tiles leave room for two waves
  // per SIMD (head_dim 128 with 32-token blocks would hold 256 registers)
  static constexpr bool PREFETCH = NK + NV <= 16;
  f32x4 k[NK];
  f32x4 v[NV];
};

template <int D, int BS>
__device__ __forceinline__ void load_f32_tile(F32Tile<D, BS>& T, const float* kt,
                                              const float* vt, int tok, int quarter, int lane) {
  typedef F32Tile<D, BS> F;
  // K [D/X][BS][X]: the lane's dims 4j .. 4j+3 of token tok, j = quarter*NK + u
#pragma unroll
  for (int u = 0; u < F::NK; ++u)
    T.k[u] = *reinterpret_cast<const f32x4*>(
        kt + ((quarter * F::NK + u) * BS + k_row<BS>(tok)) * F::X);
  // V [BS/X][D][X]: tokens 4t4 .. 4t4+3 of dim lane + 64k
#pragma unroll
  for (int t4 = 0; t4 < BS / F::X; ++t4)
#pragma unroll
    for (int k = 0; k < F::DPL; ++k)
      T.v[t4 * F::DPL + k] =
          *reinterpret_cast<const f32x4*>(vt + (t4 * D + lane + 64 * k) * F::X);
}

template <int D, int BS>
__global__ __launch_bounds__(64) void decode_part_f32(
    float* __restrict__ out, float* __restrict__ ws_o, float2* __restrict__ ws_ml,
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ block_tables, int maxb, const int32_t* __restrict__ ctx_lens,
    int max_tokens, int H_q, int H_kv, int G, int num_blocks, float scale_log2, int part,
    int maxP) {
  typedef F32Tile<D, BS> F;
  constexpr int TILE = BS * D;
  const int lane = threadIdx.x;
  const int p = blockIdx.x;
  const int qh = blockIdx.y;
  const int s = blockIdx.z;
  const int kvh = qh / G;
  const int tok = lane / F::TPL, quarter = lane % F::TPL;

  const Span sp = partition_span(ctx_lens, s, max_tokens, part, p);
  if (p >= sp.nparts) return;
  const int t0 = sp.t0, t1 = sp.t1;

  // this lane's share of q: dims 4j .. 4j+3, j = quarter*NK + u
  const int64_t row = static_cast<int64_t>(s) * H_q + qh;
  f32x4 qv[F::NK];
#pragma unroll
  for (int u = 0; u < F::NK; ++u)
    qv[u] = *reinterpret_cast<const f32x4*>(q + row * D + (quarter * F::NK + u) * F::X);

  float acc[F::DPL];
#pragma unroll
  for (int k = 0; k < F::DPL; ++k) acc[k] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int32_t* bt = block_tables + static_cast<int64_t>(s) * maxb;
  const int lb_end = (t1 + BS - 1) / BS;
  const int64_t head_off = static_cast<int64_t>(kvh) * TILE;
  const int64_t blk_stride = static_cast<int64_t>(H_kv) * TILE;

  TableWindow win;
  int lb = t0 / BS;
  if (lb < lb_end) {
    fill_window(win, bt, lb, lb_end, num_blocks, lane);
    F32Tile<D, BS> cur;
    if constexpr (F::PREFETCH) {
      const int64_t o = static_cast<int64_t>(__builtin_amdgcn_readlane(win.ids, 0)) * blk_stride;
      load_f32_tile<D, BS>(cur, kc + o + head_off, vc + o + head_off, tok, quarter, lane);
    }
    for (; lb < lb_end; ++lb) {
      F32Tile<D, BS> nxt;
      if constexpr (F::PREFETCH) {
        // request the next block before this block's arithmetic
        if (lb + 1 < lb_end) {
          if (lb + 1 >= win.lb_base + 64) fill_window(win, bt, lb + 1, lb_end, num_blocks, lane);
          const int64_t o =
              static_cast<int64_t>(__builtin_amdgcn_readlane(win.ids, lb + 1 - win.lb_base)) *
              blk_stride;
          load_f32_tile<D, BS>(nxt, kc + o + head_off, vc + o + head_off, tok, quarter, lane);
        }
      } else {
        if (lb >= win.lb_base + 64) fill_window(win, bt, lb, lb_end, num_blocks, lane);
        const int64_t o =
            static_cast<int64_t>(__builtin_amdgcn_readlane(win.ids, lb - win.lb_base)) *
            blk_stride;
        load_f32_tile<D, BS>(cur, kc + o + head_off, vc + o + head_off, tok, quarter, lane);
      }
      const int nval = (t1 - lb * BS) < BS ? (t1 - lb * BS) : BS;
      float dot = 0.f;
#pragma unroll
      for (int u = 0; u < F::NK; ++u) {
        dot = fmaf(qv[u][0], cur.k[u][0], dot);
        dot = fmaf(qv[u][1], cur.k[u][1], dot);
        dot = fmaf(qv[u][2], cur.k[u][2], dot);
        dot = fmaf(qv[u][3], cur.k[u][3], dot);
      }
#pragma unroll
      for (int mask = 1; mask < F::TPL; mask <<= 1) dot = xor_sum(dot, mask);
      const float sc = tok < nval ? dot * scale_log2 : -INFINITY;
      float bm = sc;
#pragma unroll
      for (int mask = 32; mask >= 1; mask >>= 1) bm = xor_max(bm, mask);
      const float mnew = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mnew);
      const float pe = tok < nval ? fast_exp2(sc - mnew) : 0.f;
      // each token once: the first of its lanes
      float ps = quarter == 0 ? pe : 0.f;
#pragma unroll
      for (int mask = 32; mask >= 1; mask >>= 1) ps = xor_sum(ps, mask);
      l = l * alpha + ps;
      m = mnew;
#pragma unroll
      for (int k = 0; k < F::DPL; ++k) acc[k] *= alpha;
#pragma unroll
      for (int t4 = 0; t4 < BS / F::X; ++t4) {
#pragma unroll
        for (int e = 0; e < F::X; ++e) {
          const int t = t4 * F::X + e;
          const float pt =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), t * F::TPL));
          // tokens past the fill: weight 0, and the slot's V may hold anything
          if (t < nval) {
#pragma unroll
            for (int k = 0; k < F::DPL; ++k)
              acc[k] = fmaf(pt, cur.v[t4 * F::DPL + k][e], acc[k]);
          }
        }
      }
      if constexpr (F::PREFETCH)
        if (lb + 1 < lb_end) cur = nxt;
    }
  }
  if (sp.nparts == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int k = 0; k < F::DPL; ++k) out[row * D + lane + 64 * k] = acc[k] * inv;
  } else {
    float* dst = ws_o + (row * maxP + p) * D;
#pragma unroll
    for (int k = 0; k < F::DPL; ++k) dst[lane + 64 * k] = acc[k];
    if (lane == 0) ws_ml[row * maxP + p] = make_float2(m, l);
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
// M = max m_p, L = sum 2^(m_p - M) l_p, out = sum 2^(m_p - M) o_p / L.
// One 256-thread work-group per (query head, sequence).  The weights go
// through LDS in chunks of kReduceChunk partitions; thread (lane pl, dims
// 4*d4 .. 4*d4+3) sums the partitions p = pl (mod PL) in ascending order with
// 16-byte loads, and the PL partial sums are added in lane order, so the
// result does not depend on timing.
constexpr int kReduceThreads = 256;
constexpr int kReduceChunk = 1024;

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int mask = 32; mask >= 1; mask >>= 1) v = xor_max(v, mask);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kReduceThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int mask = 32; mask >= 1; mask >>= 1) v = xor_sum(v, mask);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kReduceThreads / 64; ++i) r += red[i];
  return r;
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce(
    T* __restrict__ out, const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    const int32_t* __restrict__ ctx_lens, int max_tokens, int H_q, int part, int maxP,
    const int32_t* __restrict__ prefix_len, int prefix_nw) {
  constexpr int TPR = D / 4;                  // threads per partition row
  constexpr int PL = kReduceThreads / TPR;    // partition lanes
  __shared__ float sh_w[kReduceChunk];
  __shared__ float sh_red[kReduceThreads / 64];
  __shared__ f32x4 sh_acc[PL][TPR];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  // partials: one per chunk of the sequence's context, or, with a prefix
  // pass, one per chunk of the prefix and then one per chunk of the rest
  int ctx = ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > max_tokens ? max_tokens : ctx);
  int nchunks;
  const int plen = prefix_len ? prefix_tokens(prefix_len[s], ctx) : 0;
  if (plen > 0) {
    const int nsuf = chunks_of<NW>(ctx - plen, part);
    if (nsuf == 1) return;  // merged by the suffix pass
    nchunks = chunks_n(plen, part, prefix_nw) + nsuf;
  } else {
    nchunks = chunks_of<NW>(ctx, part);
    if (nchunks <= 1) return;
  }
  const int np = nchunks < maxP ? nchunks : maxP;
  const int64_t row = static_cast<int64_t>(s) * H_q + h;
  const float2* ml = ws_ml + row * maxP;
  const f32x4* o4 = reinterpret_cast<const f32x4*>(ws_o + row * maxP * D);

  float mx = -INFINITY;
  for (int p = tid; p < np; p += kReduceThreads) mx = fmaxf(mx, ml[p].x);
  const float M = block_max(mx, sh_red);

  const int d4 = tid % TPR, pl = tid / TPR;
  float lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < np; base += kReduceChunk) {
    const int n = np - base < kReduceChunk ? np - base : kReduceChunk;
    __syncthreads();
    for (int i = tid; i < n; i += kReduceThreads) {
      const float2 v = ml[base + i];
      const float w = fast_exp2(v.x - M);
      sh_w[i] = w;
      lsum = fmaf(w, v.y, lsum);
    }
    __syncthreads();
    const f32x4* src = o4 + static_cast<int64_t>(base) * TPR + d4;
    int i = pl;
    for (; i + 3 * PL < n; i += 4 * PL) {
      const f32x4 a0 = src[static_cast<int64_t>(i) * TPR];
      const f32x4 a1 = src[static_cast<int64_t>(i + PL) * TPR];
      const f32x4 a2 = src[static_cast<int64_t>(i + 2 * PL) * TPR];
      const f32x4 a3 = src[static_cast<int64_t>(i + 3 * PL) * TPR];
      acc += sh_w[i] * a0;
      acc += sh_w[i + PL] * a1;
      acc += sh_w[i + 2 * PL] * a2;
      acc += sh_w[i + 3 * PL] * a3;
    }
    for (; i < n; i += PL) acc += sh_w[i] * src[static_cast<int64_t>(i) * TPR];
  }
  const float L = block_sum(lsum, sh_red);
  sh_acc[pl][d4] = acc;
  __syncthreads();
  if (pl == 0) {
    f32x4 t = sh_acc[0][d4];
    for (int q = 1; q < PL; ++q) t += sh_acc[q][d4];
    const float inv = 1.f / L;
    T* dst = out + row * D + 4 * d4;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = static_cast<T>(t[r] * inv);
  }
}

inline int num_partitions(int max_ctx, int part) {
  if (part <= 0 || max_ctx <= part) return 1;
  return (max_ctx + part - 1) / part;
}

inline int num_chunks(int nparts, int per_chunk) {
  return nparts > per_chunk ? (nparts + per_chunk - 1) / per_chunk : 1;
}

struct DecodeArgs {
  const int32_t* order;  // optional sequence order (a permutation of 0..B-1)
  bool shared_kv;        // blocks may be aliased: cached loads
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
  Cascade cas;           // ngroups > 0: prefix pass + suffix pass
  int max_prefix;        // longest group prefix
  int max_members;       // largest group
  int max_rest;          // longest context part outside a group's prefix
  NewKV nkv;             // the step's appended K/V, or nulls
};

template <typename T, int D, int BS, int NW, bool NT, int MODE>
void launch_part(const DecodeArgs& a, int maxC, int ws_stride, int nitems) {
  const int n_hg = (a.G + 15) / 16;
  const int64_t grid = static_cast<int64_t>(maxC) * a.H_kv * n_hg * nitems;
  if (grid == 0) return;
  hipLaunchKernelGGL((decode_part_mfma<T, D, BS, NW, NT, MODE>),
                     dim3(static_cast<unsigned>(grid)), dim3(64 * NW), 0, a.st,
                     static_cast<T*>(a.out), a.ws_o, a.ws_ml, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.kc), static_cast<const T*>(a.vc), a.bt, a.maxb,
                     a.lens, a.order, a.B, a.max_tokens, a.H_q, a.H_kv, a.G, n_hg, a.num_blocks,
                     a.scale_log2, a.part, maxC, ws_stride, a.cas, a.nkv);
}

// Partial slots per (sequence, query head) row.
inline int host_chunks(int n, int part, int nw) {
  if (part <= 0) return 1;
  const int nparts = (n + part - 1) / part;
  return nparts > nw ? (nparts + nw - 1) / nw : 1;
}

template <typename T, int D, int BS, int NW>
void launch_mfma_nw(const DecodeArgs& a) {
  const int maxC = num_chunks(a.maxP, NW);
  if (a.cas.ngroups == 0) {
    if (a.shared_kv)
      launch_part<T, D, BS, NW, false, kPlain>(a, maxC, maxC, a.B);
    else
      launch_part<T, D, BS, NW, true, kPlain>(a, maxC, maxC, a.B);
    if (maxC > 1)
      hipLaunchKernelGGL((decode_reduce<T, D, NW>), dim3(a.H_q, a.B), dim3(kReduceThreads), 0,
                         a.st, static_cast<T*>(a.out), a.ws_o, a.ws_ml, a.lens, a.max_tokens,
                         a.H_q, a.part, maxC, nullptr, 0);
    return;
  }
  // prefix pass (groups re-read the same blocks: cached loads), then the rest
  // of every sequence, then the merge; row stride maxC + 1 slots
  // (the suffixes are mostly private blocks: streaming loads)
  // (the slot stride counts prefix chunks of NWP waves: with more waves per
  // chunk a row has no more chunks, so the stride, and the workspace size
  // that assumes it, stay bounds)
  constexpr int NWP = PrefixNW<NW>::value, NWP2 = Prefix2NW<NW>::value;
  const bool two = a.max_members * a.G > 16;
  DecodeArgs b = a;
  b.cas.prefix_nw = two ? NWP2 : NWP;
  const int stride = host_chunks(a.max_tokens, a.part, NWP) + 1;
  const int cp = host_chunks(a.max_prefix, a.part, b.cas.prefix_nw);
  // A family wider than one column group (32 / G members) spans several
  // groups that re-read its blocks: cached loads, XCD-aware order.  When the
  // largest group is smaller than that, every group is a whole family and
  // each prefix block is read once: streaming loads, as in the plain pass.
  const bool reread = a.max_members >= 32 / a.G;
  if (two) {
    if (reread)
      launch_part<T, D, BS, NWP2, false, kPrefix2>(b, cp, stride, a.cas.ngroups);
    else
      launch_part<T, D, BS, NWP2, true, kPrefix2>(b, cp, stride, a.cas.ngroups);
  } else {
    if (reread)
      launch_part<T, D, BS, NWP, false, kPrefix>(b, cp, stride, a.cas.ngroups);
    else
      launch_part<T, D, BS, NWP, true, kPrefix>(b, cp, stride, a.cas.ngroups);
  }
  launch_part<T, D, BS, NW, true, kSuffix>(b, maxC, stride, a.B);
  if (host_chunks(a.max_rest, a.part, NW) > 1)  // some rest takes several chunks
    hipLaunchKernelGGL((decode_reduce<T, D, NW>), dim3(a.H_q, a.B), dim3(kReduceThreads), 0,
                       a.st, static_cast<T*>(a.out), a.ws_o, a.ws_ml, a.lens, a.max_tokens,
                       a.H_q, a.part, stride, a.cas.prefix_len, b.cas.prefix_nw);
}

// Waves per work-group for a partition size (see kChunkTokens).
inline int waves_per_group(int part) {
  if (part <= 0) return 8;
  const int want = kChunkTokens / part;
  return want >= 8 ? 8 : want >= 4 ? 4 : want >= 2 ? 2 : 1;
}

// Waves per work-group of the plain or suffix pass: 6 instead of 4 for long
// contexts without a cascade (see kLongParts).
inline int pass_waves(int part, int maxP, bool cascade) {
  const int nw = waves_per_group(part);
  return nw == 4 && !cascade && maxP >= kLongParts ? 6 : nw;
}

template <typename T, int D, int BS>
void launch_mfma(const DecodeArgs& a) {
  switch (pass_waves(a.part, a.maxP, a.cas.ngroups > 0)) {
    case 8: launch_mfma_nw<T, D, BS, 8>(a); break;
    case 6: launch_mfma_nw<T, D, BS, 6>(a); break;
    case 4: launch_mfma_nw<T, D, BS, 4>(a); break;
    case 2: launch_mfma_nw<T, D, BS, 2>(a); break;
    default: launch_mfma_nw<T, D, BS, 1>(a); break;
  }
}

template <int D, int BS>
void launch_f32(const DecodeArgs& a) {
  hipLaunchKernelGGL((decode_part_f32<D, BS>), dim3(a.maxP, a.H_q, a.B), dim3(64), 0, a.st,
                     static_cast<float*>(a.out), a.ws_o, a.ws_ml, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.kc), static_cast<const float*>(a.vc), a.bt,
                     a.maxb, a.lens, a.max_tokens, a.H_q, a.H_kv, a.G, a.num_blocks,
                     a.scale_log2, a.part, a.maxP);
  if (a.maxP > 1)
    hipLaunchKernelGGL((decode_reduce<float, D, 1>), dim3(a.H_q, a.B), dim3(kReduceThreads), 0,
                       a.st, static_cast<float*>(a.out), a.ws_o, a.ws_ml, a.lens, a.max_tokens,
                       a.H_q, a.part, a.maxP, nullptr, 0);
}

template <typename T>
void dispatch_mfma(const DecodeArgs& a, int D, int BS) {
  if (D == 64 && BS == 16) launch_mfma<T, 64, 16>(a);
  else if (D == 64 && BS == 32) launch_mfma<T, 64, 32>(a);
  else if (D == 128 && BS == 16) launch_mfma<T, 128, 16>(a);
  else launch_mfma<T, 128, 32>(a);
}

// Partial slots per (sequence, query head) row that a decode writes: one per
// partition on the fp32 path, one per chunk of the plain pass, and with a
// cascade the prefix chunks (counted at the one-tile pass's wave count, an
// upper bound) plus one for the rest; 0 when no row has more than one.
inline int workspace_slots(int dtype, int max_context_len, int partition_size, bool cascade) {
  const int maxP = num_partitions(max_context_len, partition_size);
  const int part = maxP > 1 ? partition_size : 0;
  if (cascade)
    return host_chunks(max_context_len, part, std::min(waves_per_group(part), kPrefixWaves)) + 1;
  if (dtype == PA_F32) return maxP > 1 ? maxP : 0;
  const int maxC = num_chunks(maxP, pass_waves(part, maxP, false));
  return maxC > 1 ? maxC : 0;
}

// Workspace layout: fp32 o[rows][slots][head_dim] (256-byte aligned size),
// then float2 (m, l)[rows][slots].
struct WsLayout {
  size_t o_bytes, total;
};
inline WsLayout workspace_layout(size_t rows, int slots, int head_dim) {
  WsLayout w{0, 0};
  if (slots <= 0) return w;
  const size_t n = rows * static_cast<size_t>(slots);
  w.o_bytes = (n * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
  w.total = w.o_bytes + n * sizeof(float2);
  return w;
}


}  // namespace pa

using namespace pa;

PA_EXPORT size_t pa_decode_cascade_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                                  int max_context_len, int partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  const int maxP = num_partitions(max_context_len, partition_size);
  const int part = maxP > 1 ? partition_size : 0;
  const int nw = std::min(waves_per_group(part), kPrefixWaves);
  const int stride = host_chunks(max_context_len, part, nw) + 1;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * stride;
  const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return o_bytes + rows * sizeof(float2);
}

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

namespace pa {

pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int num_seqs, int max_context_len,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float scale, int partition_size, void* workspace,
                      size_t workspace_bytes, int dtype, int flags, const int32_t* order,
                      void* stream, const CascadePlan* plan, const NewKV* nkv) {
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (flags & ~PA_DECODE_SHARED_KV) return PA_ERR_INVALID;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_context_len < 0 || max_blocks_per_seq < 0 || partition_size < 0)
    return PA_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (partition_size % 32 != 0) return PA_ERR_INVALID;
  // the fp16 / bf16 path takes the running max of unscaled scores
  if (!(scale > 0.f) || !std::isfinite(scale)) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_context_len) >
      static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID;
  if (num_seqs > 65535 || num_q_heads > 65535) return PA_ERR_INVALID;
  // the cascade runs on the fp16 / bf16 path for up to 16 query heads per KV head
  const bool cascade = plan && plan->ngroups > 0 && dtype != PA_F32 &&
                       num_q_heads / num_kv_heads <= 16;
  if (cascade && (!plan->prefix_len || !plan->groups || !plan->members || plan->ngroups < 0 ||
                  plan->max_prefix < 0 || plan->max_prefix > max_context_len ||
                  plan->max_members < 1 ||
                  plan->max_members * (num_q_heads / num_kv_heads) > 32 ||
                  plan->max_rest < 0 || plan->max_rest > max_context_len))
    return PA_ERR_INVALID;
  // exactly the partial slots this call writes (pa_decode_workspace_size and
  // pa_decode_cascade_workspace_size give bounds of it)
  const WsLayout ws = workspace_layout(static_cast<size_t>(num_seqs) * num_q_heads,
                                       workspace_slots(dtype, max_context_len, partition_size,
                                                       cascade),
                                       head_dim);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total || !aligned16(workspace)))
    return PA_ERR_INVALID;

  DecodeArgs a;
  a.order = order;
  a.shared_kv = (flags & PA_DECODE_SHARED_KV) != 0;
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
  a.cas = Cascade{nullptr, nullptr, nullptr, 0, 0};
  a.max_prefix = 0;
  a.max_members = 0;
  a.max_rest = 0;
  a.nkv = NewKV{nullptr, nullptr};
  if (nkv && nkv->k && nkv->v && dtype != PA_F32) {
    if (!aligned16(nkv->k) || !aligned16(nkv->v)) return PA_ERR_INVALID;
    a.nkv = *nkv;
  }
  if (cascade) {
    a.cas = Cascade{plan->prefix_len, plan->groups, plan->members, plan->ngroups, 0};
    a.max_prefix = plan->max_prefix;
    a.max_members = plan->max_members;
    a.max_rest = plan->max_rest;
  }
  if (ws.total > 0) {
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + ws.o_bytes);
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

}  // namespace pa

PA_EXPORT pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                              int max_context_len, int num_q_heads, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, float scale,
                              int partition_size, void* workspace, size_t workspace_bytes,
                              int dtype, int flags, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, workspace, workspace_bytes, dtype, flags,
                     seq_order, stream, nullptr, nullptr);
}

PA_EXPORT pa_status pa_decode_cascade(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens,
                                      const int32_t* seq_order, int num_seqs, int max_context_len,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, float scale,
                                      int partition_size, const int32_t* prefix_len,
                                      const int32_t* groups, const int32_t* members,
                                      int num_groups, int max_prefix, int max_members,
                                      int max_rest, void* workspace, size_t workspace_bytes,
                                      int dtype, int flags, void* stream) {
  if (num_groups < 0) return PA_ERR_INVALID;
  const CascadePlan plan{prefix_len, groups, members, num_groups, max_prefix, max_members,
                         max_rest};
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, workspace, workspace_bytes, dtype, flags,
                     seq_order, stream, &plan, nullptr);
}

// ---------------------------------------------------------------------------
// pa_decode_noalloc: pa_decode with its split-K partials in a fixed device
// array owned by the library, for callers that cannot allocate.
// ---------------------------------------------------------------------------

namespace pa {

constexpr size_t kScratchBytes = static_cast<size_t>(PA_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

}  // namespace pa

// One copy per GPU the library runs on, held until the process ends.  Host
// code never passes this name to a kernel: it stands for the host-side
// shadow, not the device address, which scratch_address() looks up.
static __device__ __align__(256) unsigned char scratch[pa::kScratchBytes];

namespace pa {
namespace {

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
pa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

PA_EXPORT pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens,
                                      const int32_t* seq_order, int num_seqs,
                                      int max_context_len, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks, float scale,
                                      int partition_size, int dtype, int flags, void* stream) {
  // the partials this call writes, before anything touches the device
  size_t need = 0;
  if (num_seqs > 0 && num_q_heads > 0 && head_dim > 0 && max_context_len >= 0 &&
      partition_size >= 0)
    need = workspace_layout(static_cast<size_t>(num_seqs) * num_q_heads,
                            workspace_slots(dtype, max_context_len, partition_size, false),
                            head_dim)
               .total;
  if (need > kScratchBytes) return PA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    const pa_status st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, ws, ws ? kScratchBytes : 0, dtype, flags,
                     seq_order, stream, nullptr, nullptr);
}
