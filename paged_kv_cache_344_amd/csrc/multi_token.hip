// multi_token.hip - the gfx950 kernel behind pa_multi_token: attention for several new
// tokens per sequence over the paged cache (a prompt chunk, or draft tokens to verify).
//
// Pages cited (title, site): [ASP] "PagedAttention" awesome-system-papers, sections
// 实现要点 (continuous batching adds sequences every step, so their prompt tokens are
// attended through the same block tables) and 已知局限 (speculative decoding over the
// paged cache); 引用本概念的论文 (the cache serves the scaled dot-product attention of
// "Attention Is All You Need", where a token sees itself and every earlier token);
// [RK] "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?" news.rkmt.cn, 块表.
//
// What is computed.  Sequence s has L tokens cached, the last n of them new; new token
// j sits at position c + j (c = L - n) and attends to positions 0 .. c + j.  Rows of
// the problem are (new token, query head) pairs; the G query heads of one KV head
// share every K/V byte, so one KV head's rows form a dense (rows x tokens) problem,
// which is where the matrix cores pay.
//
// Work.  A workgroup (4 waves) owns 128 consecutive rows of one (sequence, KV head):
// row r is new token r / G, query head r % G of the group.  Each wave holds 32 rows as
// two 16-row MFMA tiles.  The workgroup walks the sequence's tokens in 32-token chunks
// up to the last position its rows may see; each chunk's K and V are gathered through
// the block table once into LDS (double-buffered, the next chunk's loads in flight while
// the current one is computed) and read there by all four waves.
//
// MFMA layouts (as in the decode kernel, rows of the problem on the N side):
//   logits^T = K (32 tokens x D) . Q^T (D x 16 rows), two 16-token tiles per chunk
//   taking tokens {8i..8i+3} and {8i+4..8i+7}, so lane (row c, quad i) ends up holding
//   tokens 8i..8i+7 of row c: exactly the B operand (P^T) of
//   O^T += V^T (16 dims x 32 tokens) . P^T (32 tokens x 16 rows).
// K is stored in LDS in that MFMA row order ([tile][row][D], padded), V dimension-major
// ([D][32 tokens], padded), so every operand is one 16-byte LDS read per lane.
//
// Masking.  Positions past the causal limit of a row are removed by select (-inf
// before the max, weight 0).  Positions at or past L may hold anything, so they are
// written to LDS as zeros and never multiplied.
//
// Precision.  Products accumulate in fp32.  The softmax weights enter the second product
// as a hi + lo pair for bf16 (its 8 significant bits alone would show next to the
// output's own rounding), rounded once for fp16, and exactly for fp32; the sum that
// normalises them is kept in fp32.
//
// Context split.  With few (row tile, KV head, sequence) triples, as when a few draft
// tokens per sequence are verified against long contexts, the tokens of each sequence
// are cut into partitions of part_tokens positions, one workgroup each; every
// workgroup leaves its rows' running maximum, sum and unnormalised output in a
// workspace, and a second launch combines them with log-sum-exp weights.
//
// Launch.  One workgroup per (row tile, partition, KV head, sequence).  Workgroups are dispatched
// to the eight XCDs in turn; the numbering deals whole (sequence, KV head) groups to
// the XCDs round-robin, so that the row tiles of a group share their XCD's L2 copy of
// the K/V they all read, and every XCD gets a share of every sequence.
#include <math.h>

#include <type_traits>

#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define AS4 __attribute__((address_space(4)))  // constant address space: scalar loads

constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int NTILE = 2;                    // 16-row MFMA tiles per wave
constexpr int ROWS = WAVES * NTILE * 16;    // rows of one workgroup
constexpr int CH = 32;                      // tokens per chunk
constexpr int XCDS = 8;

template <typename T>
struct V8;
template <>
struct V8<__bf16> {
  typedef bf16x8 type;
};
template <>
struct V8<_Float16> {
  typedef f16x8 type;
};

__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes c, c + 16, c + 32 and c + 48 (the four quads) hold parts of the same row: reduce
// over them with the gfx950 lane-swap instructions (VALU, no LDS round trip).
__device__ __forceinline__ float vmax(float a, float b) {  // v_max_f32, no canonicalisation
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(a), "v"(b));
  return m;
}
__device__ __forceinline__ float max_over_quads(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));  // lanes l and l ^ 32
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));  // and l ^ 16
}
__device__ __forceinline__ float sum_over_quads(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// maximum of eight values as three v_max3 and one v_max (no NaN canonicalisation steps)
__device__ __forceinline__ float max8(const float (&z)[8]) {
  float a, b, c, m;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(a) : "v"(z[0]), "v"(z[1]), "v"(z[2]));
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(b) : "v"(z[3]), "v"(z[4]), "v"(z[5]));
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(c) : "v"(a), "v"(b), "v"(z[6]));
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(c), "v"(z[7]));
  return m;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// eight weights as MFMA operands of a 16-bit type: hi = nearest T, and (bf16 only)
// lo = nearest T to the remainder, converted two at a time
template <typename T>
__device__ __forceinline__ void split_weights(const float (&p)[8], u32x4& hi, u32x4& lo) {
  typedef typename std::conditional<std::is_same<T, __bf16>::value, bf16x2, f16x2>::type T2;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const T2 h = __builtin_convertvector((f32x2){p[2 * k], p[2 * k + 1]}, T2);
    hi[k] = __builtin_bit_cast(uint32_t, h);
    if constexpr (std::is_same<T, __bf16>::value) {
      // a bf16 is the upper half of an fp32: widen both halves exactly, take the rest
      const float h0 = __uint_as_float(hi[k] << 16), h1 = __uint_as_float(hi[k] & 0xFFFF0000u);
      const T2 l = __builtin_convertvector((f32x2){p[2 * k] - h0, p[2 * k + 1] - h1}, T2);
      lo[k] = __builtin_bit_cast(uint32_t, l);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    T t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (T)v[e];
    *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, t);
  }
}

template <typename T, int D, int BS>
struct Shape {
  static constexpr int E = sizeof(T);
  static constexpr int EPL = 16 / E;                 // elements per 16 bytes
  static constexpr int KL = D * E / 64;              // 16-byte operand reads per key row
  static constexpr int NT = D / 16;                  // 16-dimension output tiles
  static constexpr int KROW = D + EPL;               // LDS pitch of a key row (elements)
  static constexpr int VROW = CH + EPL;              // LDS pitch of a value row
  static constexpr int KSEG = D * E / 16;            // 16-byte pieces of a key row
  static constexpr int KP = CH * KSEG / THREADS;     // key pieces per thread per chunk
  static constexpr int VPE = EPL < BS ? EPL : BS;    // tokens per value piece
  static constexpr int VSEG = CH / VPE;              // value pieces per dimension
  static constexpr int VP = D * VSEG / THREADS;      // value pieces per thread per chunk
  static_assert(KP >= 1 && VP >= 1, "chunk pieces must cover the workgroup");
  typedef typename std::conditional<VPE * E == 16, u32x4, u32x2>::type VPiece;
};

// rows of the LDS key tile are in MFMA order: token t = 8a + 4q + b sits at 16q + 4a + b
__device__ __forceinline__ int krow_of(int t) { return 16 * ((t >> 2) & 1) + 4 * (t >> 3) + (t & 3); }

template <typename T, int D, int BS>
__global__ __launch_bounds__(THREADS, sizeof(T) == 2 ? 2 : 1) void multi_token_kernel(MultiTokenParams P) {
  typedef Shape<T, D, BS> SH;
  constexpr int KL = SH::KL, NT = SH::NT, EPL = SH::EPL;
  typedef typename SH::VPiece VPiece;

  __shared__ __attribute__((aligned(16))) T sk[2][CH * SH::KROW];
  __shared__ __attribute__((aligned(16))) T sv[2][D * SH::VROW];

  // ---- which (row tile, context partition, KV head, sequence): (sequence, KV head)
  // groups are dealt to the XCDs in turn, and every row tile and partition of a group
  // runs on its group's XCD
  const int per_group = P.row_tiles * P.parts;
  const int xcd = (int)(blockIdx.x % XCDS);
  const int idx = (int)(blockIdx.x / XCDS);
  const int group = (idx / per_group) * XCDS + xcd;
  if (group >= P.num_kv_heads * P.num_seqs) return;
  const int x = idx % P.row_tiles;
  const int part = (idx % per_group) / P.row_tiles;
  const int g = group % P.num_kv_heads;
  const int s = group / P.num_kv_heads;
  const bool split = P.parts > 1;

  const int G = P.group, Hq = P.num_q_heads;
  const int q0 = P.query_start[s], q1 = P.query_start[s + 1];
  const int n = q1 - q0;
  // rows that cannot be placed inside out[0 .. T) are never written
  if (q0 < 0 || n < 0 || q1 > P.num_tokens) return;
  const int nrows = n * G;
  const int R0 = x * ROWS;
  if (R0 >= nrows) return;
  const int rend = min(nrows, R0 + ROWS);
  const int L = P.seq_lens[s];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int quad = lane >> 4;

  if (L > P.max_tokens || n > L) {  // a length the table cannot hold: NaN rows
    if (split) return;                // (the merge writes them)
    for (int i = tid; i < (rend - R0) * D; i += THREADS) {
      const int rr = R0 + i / D;
      const int64_t row = (int64_t)(q0 + rr / G) * Hq + g * G + rr % G;
      ((T*)P.out)[row * D + i % D] = (T)__builtin_nanf("");
    }
    return;
  }
  const int ctx = L - n;
  const int lim_lo = ctx + R0 / G;          // the earliest causal limit among these rows
  const int lim_hi = ctx + (rend - 1) / G;  // the latest
  // this workgroup's chunks: c_lo .. nch-1 of the 0 .. lim_hi / CH its rows may see
  const int c_lo = part * (P.part_tokens / CH);
  const int nch = split ? min(lim_hi / CH + 1, c_lo + P.part_tokens / CH) : lim_hi / CH + 1;
  if (c_lo >= nch) return;  // a partition past these rows' positions: the merge skips it
  const int last_blk = (L - 1) / BS;

  const uint32_t nblk32 = (uint32_t)min(P.num_blocks, (int64_t)0x7fffffff);
  const int64_t tile = (int64_t)BS * D;
  const int64_t blk_stride = (int64_t)P.num_kv_heads * tile;
  const T* kbase = (const T*)P.k_cache + (int64_t)g * tile;
  const T* vbase = (const T*)P.v_cache + (int64_t)g * tile;
  const int32_t* tbl = P.block_tables + (int64_t)s * P.max_blocks;

  // ---- this lane's rows: query fragments and causal limits.  A negative scale is
  // applied as |scale| to queries with their sign bits flipped (exact), so that the
  // largest logit is the largest raw dot product.
  const float sc = fabsf(P.scale_log2);
  const uint32_t qsign = P.scale_log2 < 0.f ? (sizeof(T) == 2 ? 0x80008000u : 0x80000000u) : 0u;
  u32x4 qf[NTILE][KL];
  int lim[NTILE];
  bool rvalid[NTILE];
  int64_t orow[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int rr = R0 + wave * (NTILE * 16) + t * 16 + col;
    rvalid[t] = rr < rend;
    const int rc = min(rr, rend - 1);
    const int j = rc / G;
    lim[t] = ctx + j;
    orow[t] = (int64_t)(q0 + j) * Hq + g * G + rc % G;
    const T* qp = (const T*)P.q + orow[t] * D + quad * EPL;
#pragma unroll
    for (int c = 0; c < KL; ++c)
      qf[t][c] = rvalid[t] ? (*reinterpret_cast<const u32x4*>(qp + c * 4 * EPL) ^ qsign)
                           : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- chunk loading, block ids one chunk ahead of the data.  Key piece p (of a
  // thread's KP) is token p / KSEG of the chunk, 16-byte segment p % KSEG of its row;
  // value piece p is dimension p % D, tokens VPE * (p / D) onwards.  One wave-wide load
  // instruction thus covers whole token groups, and the physical block it reads is the
  // same for all its lanes: one scalar table read per instruction, and the block's
  // address is formed in scalar registers.  Only 8-token key groups at block size 4
  // span two blocks; there each lane picks one of the two.
  constexpr int TPI = 64 / SH::KSEG;              // tokens under one wave-wide key load
  constexpr int NBK = TPI > BS ? TPI / BS : 1;    // blocks those tokens span
  static_assert(NBK <= 2, "a key load spans at most two blocks");
  const int32_t AS4* tbls = (const int32_t AS4*)tbl;
  int bad = 0;
  int kid[SH::KP][NBK], vid[SH::VP];
  u32x4 kr[SH::KP];
  VPiece vr[SH::VP];
  // table reads go out one chunk before their ids are used, and are checked only then,
  // so that the wait for them falls long after they arrived
  auto block_id = [&](int j) { return tbls[min(j, last_blk)]; };
  auto checked = [&](int id) {  // ids outside the pool -> 0, and the workgroup's rows NaN
    const bool ok = (uint32_t)id < nblk32;
    bad |= !ok;
    return ok ? id : 0;
  };
  auto load_ids = [&](int c, int (&ki)[SH::KP][NBK], int (&vi)[SH::VP]) {
    const int t0 = c * CH;
#pragma unroll
    for (int i = 0; i < SH::KP; ++i) {
      const int j = (t0 + (64 * wave + THREADS * i) / SH::KSEG) / BS;
#pragma unroll
      for (int u = 0; u < NBK; ++u) ki[i][u] = block_id(j + u);
    }
#pragma unroll
    for (int i = 0; i < SH::VP; ++i)
      vi[i] = block_id((t0 + ((64 * wave + THREADS * i) / D) * SH::VPE) / BS);
  };
  auto load_data = [&]() {
#pragma unroll
    for (int i = 0; i < SH::KP; ++i) {
      const int p = tid + THREADS * i;
      const int t = p / SH::KSEG;  // (t0 + t) % BS == t % BS: chunks start on block edges
      int id = checked(kid[i][0]);
      if constexpr (NBK == 2) {
        const int id1 = checked(kid[i][1]);
        id = ((t % TPI) >= BS) ? id1 : id;
      }
      const T* blk = kbase + (int64_t)id * blk_stride;
      kr[i] = *reinterpret_cast<const u32x4*>(blk + (t % BS) * D + (p % SH::KSEG) * EPL);
    }
#pragma unroll
    for (int i = 0; i < SH::VP; ++i) {
      const int p = tid + THREADS * i;
      const int tk = (p / D) * SH::VPE;
      const T* blk = vbase + (int64_t)checked(vid[i]) * blk_stride;
      vr[i] = *reinterpret_cast<const VPiece*>(blk + (p % D) * BS + tk % BS);
    }
  };
  auto store_lds = [&](int c, int buf) {
    const int t0 = c * CH;
#pragma unroll
    for (int i = 0; i < SH::KP; ++i) {
      const int p = tid + THREADS * i;
      const int t = p / SH::KSEG;
      const u32x4 v = (t0 + t < L) ? kr[i] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&sk[buf][krow_of(t) * SH::KROW + (p % SH::KSEG) * EPL]) = v;
    }
#pragma unroll
    for (int i = 0; i < SH::VP; ++i) {
      const int p = tid + THREADS * i;
      const int tk = (p / D) * SH::VPE;
      VPiece v = vr[i];
      if (t0 + tk + SH::VPE > L) {  // values at or past L may be NaN: zero them
        constexpr int W = sizeof(VPiece) / 4;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          if constexpr (sizeof(T) == 2) {
            const int e = t0 + tk + 2 * w;
            v[w] &= (e < L ? 0x0000FFFFu : 0u) | (e + 1 < L ? 0xFFFF0000u : 0u);
          } else {
            v[w] = (t0 + tk + w < L) ? v[w] : 0u;
          }
        }
      }
      *reinterpret_cast<VPiece*>(&sv[buf][(p % D) * SH::VROW + tk]) = v;
    }
  };

  float m_run[NTILE], l_run[NTILE];
  f32x4 acc[NTILE][NT];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) acc[t][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One chunk: logits for both row tiles (the key operand read once for both), then per
  // tile the softmax and the weighted sum.  Only a chunk that crosses the causal limit of
  // some row of the workgroup is masked.
  auto compute = [&](int c, int buf) {
    const int t0 = c * CH;
    const bool masked = t0 + CH - 1 > lim_lo;  // uniform
    // logits^T tiles a (tokens 8i..8i+3) and b (8i+4..8i+7); A read once for both row tiles
    f32x4 sa[NTILE], sb[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) sa[t] = sb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const T* ka = &sk[buf][col * SH::KROW + quad * EPL];
    const T* kb = &sk[buf][(16 + col) * SH::KROW + quad * EPL];
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(ka + k * 4 * EPL);
      const u32x4 b = *reinterpret_cast<const u32x4*>(kb + k * 4 * EPL);
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        if constexpr (sizeof(T) == 2) {
          typedef typename V8<T>::type VT;
          sa[t] = mma16(__builtin_bit_cast(VT, a), __builtin_bit_cast(VT, qf[t][k]), sa[t]);
          sb[t] = mma16(__builtin_bit_cast(VT, b), __builtin_bit_cast(VT, qf[t][k]), sb[t]);
        } else {
          const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
          const f32x4 qv = __builtin_bit_cast(f32x4, qf[t][k]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sa[t] = mma4(af[e], qv[e], sa[t]);
            sb[t] = mma4(bf[e], qv[e], sb[t]);
          }
        }
      }
    }
    // per row tile: softmax of the chunk, then its weighted sum
    const int tfirst = t0 + 8 * quad;
    const T* vrow = &sv[buf][col * SH::VROW + 8 * quad];  // dimension 16nn + col, tokens 8quad..
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      float z[8];  // raw dot products; the scale is applied inside the exponent
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[e] = sa[t][e];
        z[4 + e] = sb[t][e];
      }
      if (masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (tfirst + e <= lim[t]) ? z[e] : -INFINITY;
      }
      const float cm = max_over_quads(max8(z));
      // a row with every position of this chunk masked keeps its maximum (max(m, -inf)
      // = m); while it has seen no position at all (a partition that starts past its
      // causal limit) the maximum stays -inf and is taken as 0 in the exponents, so that
      // its weights and rescale factor are exp2(-inf) = 0, never exp2(-inf + inf)
      const float m_new = fmaxf(m_run[t], cm * sc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(m_run[t] - m_use);
      float pr[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = exp2_fast(__builtin_fmaf(z[e], sc, -m_use));
      if (masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = (tfirst + e <= lim[t]) ? pr[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) psum += pr[e];
      l_run[t] = l_run[t] * alpha + psum;
      m_run[t] = m_new;
      // after the first chunks the running maximum rarely moves: rescale only when it
      // moved for some row of this wave
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) acc[t][nn] *= alpha;
      }
      if constexpr (sizeof(T) == 2) {
        // bf16 keeps 8 significant bits: the weights go in as a hi + lo pair (two
        // MFMAs), about fp32 accuracy, so that the output's own rounding is the only
        // visible error; fp16's 11 bits need one rounding only
        typedef typename V8<T>::type VT;
        u32x4 phi, plo;
        split_weights<T>(pr, phi, plo);
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const VT vv = *reinterpret_cast<const VT*>(vrow + 16 * nn * SH::VROW);
          acc[t][nn] = mma16(vv, __builtin_bit_cast(VT, phi), acc[t][nn]);
          if constexpr (std::is_same<T, __bf16>::value)
            acc[t][nn] = mma16(vv, __builtin_bit_cast(VT, plo), acc[t][nn]);
        }
      } else {
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(vrow + 16 * nn * SH::VROW);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(vrow + 16 * nn * SH::VROW + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][nn] = mma4(lo[e], pr[e], acc[t][nn]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][nn] = mma4(hi[e], pr[4 + e], acc[t][nn]);
        }
      }
    }
  };

  // ---- the chunk pipeline over chunks c_lo .. nch-1
  load_ids(c_lo, kid, vid);
  load_data();
  store_lds(c_lo, c_lo & 1);
  if (c_lo + 1 < nch) load_ids(c_lo + 1, kid, vid);
  __syncthreads();
  for (int c = c_lo; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) load_data();
    int kid2[SH::KP][NBK], vid2[SH::VP];
    if (c + 2 < nch) load_ids(c + 2, kid2, vid2);
    compute(c, buf);
    if (c + 1 < nch) store_lds(c + 1, buf ^ 1);
    if (c + 2 < nch) {
#pragma unroll
      for (int i = 0; i < SH::KP; ++i)
#pragma unroll
        for (int u = 0; u < NBK; ++u) kid[i][u] = kid2[i][u];
#pragma unroll
      for (int i = 0; i < SH::VP; ++i) vid[i] = vid2[i];
    }
    __syncthreads();
  }
  bad = __syncthreads_or(bad);

  if (split) {
    // this partition's partial rows for the merge: running maximum (log2 units), sum
    // and unnormalised output; a bad table entry makes them NaN
    const int64_t tile0 =
        ((((int64_t)s * P.num_kv_heads + g) * P.row_tiles + x) * P.parts + part) * P.part_rows;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const float l = sum_over_quads(l_run[t]);
      if (!rvalid[t]) continue;
      const int64_t r = tile0 + wave * (NTILE * 16) + t * 16 + col;
      float* po = P.part_o + r * D + 4 * quad;
#pragma unroll
      for (int nn = 0; nn < NT; ++nn)
        *reinterpret_cast<f32x4*>(po + 16 * nn) = bad ? f32x4{nan, nan, nan, nan} : acc[t][nn];
      if (quad == 0)
        *reinterpret_cast<f32x2*>(P.part_ml + 2 * r) = bad ? f32x2{nan, nan} : f32x2{m_run[t], l};
    }
    return;
  }

  // ---- normalise and store
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const float l = sum_over_quads(l_run[t]);
    if (!rvalid[t]) continue;
    T* o = (T*)P.out + orow[t] * D + 4 * quad;
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) {
      f32x4 v = acc[t][nn] / l;
      if (bad) v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      store4(o + 16 * nn, v);
    }
  }
}

// The merge after a split launch: one workgroup per (row tile, KV head, sequence)
// combines each row's partitions with log-sum-exp weights, in partition order, and
// writes the output row (NaN rows for a length the table cannot hold).  Partitions that
// start past the tile's last causal limit were skipped by the main kernel; the first
// partition always holds position 0, which every row sees.
template <typename T, int D>
__global__ __launch_bounds__(THREADS) void multi_token_merge_kernel(MultiTokenParams P) {
  const int x = (int)(blockIdx.x % P.row_tiles);
  const int group = (int)(blockIdx.x / P.row_tiles);
  const int g = group % P.num_kv_heads;
  const int s = group / P.num_kv_heads;
  const int G = P.group, Hq = P.num_q_heads;
  const int q0 = P.query_start[s], q1 = P.query_start[s + 1];
  const int n = q1 - q0;
  if (q0 < 0 || n < 0 || q1 > P.num_tokens) return;
  const int R0 = x * ROWS;
  const int rend = min(n * G, R0 + ROWS);
  if (R0 >= rend) return;
  const int L = P.seq_lens[s];
  const bool invalid = L > P.max_tokens || n > L;
  const int lim_hi = L - n + (rend - 1) / G;
  const int used = min(P.parts, (lim_hi / CH) / (P.part_tokens / CH) + 1);
  const int64_t tile0 = (((int64_t)s * P.num_kv_heads + g) * P.row_tiles + x) * P.parts * P.part_rows;
  const int64_t pstride = P.part_rows;
  for (int it = threadIdx.x; it < (rend - R0) * (D / 4); it += THREADS) {
    const int r = it / (D / 4);
    const int d4 = (it - r * (D / 4)) * 4;
    const int rr = R0 + r;
    T* o = (T*)P.out + ((int64_t)(q0 + rr / G) * Hq + g * G + rr % G) * D + d4;
    if (invalid) {
      const float nan = __builtin_nanf("");
      store4(o, f32x4{nan, nan, nan, nan});
      continue;
    }
    float M = -INFINITY;
    for (int p = 0; p < used; ++p) M = fmaxf(M, P.part_ml[2 * (tile0 + p * pstride + r)]);
    float Ls = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    bool nan_seen = false;
    for (int p = 0; p < used; ++p) {
      const int64_t pr = tile0 + p * pstride + r;
      const f32x2 ml = *reinterpret_cast<const f32x2*>(P.part_ml + 2 * pr);
      nan_seen |= ml[0] != ml[0];
      const float w = exp2_fast(ml[0] - M);  // 0 for a partition none of whose positions the row sees
      Ls += w * ml[1];
      O += w * *reinterpret_cast<const f32x4*>(P.part_o + pr * D + d4);
    }
    const float nan = __builtin_nanf("");
    store4(o, nan_seen ? f32x4{nan, nan, nan, nan} : O / Ls);
  }
}

template <typename T, int D>
const void* mt_bs(int bs) {
  switch (bs) {
    case 4: return (const void*)multi_token_kernel<T, D, 4>;
    case 8: return (const void*)multi_token_kernel<T, D, 8>;
    case 16: return (const void*)multi_token_kernel<T, D, 16>;
    case 32: return (const void*)multi_token_kernel<T, D, 32>;
  }
  return nullptr;
}

template <typename T>
const void* mt_d(int d, int bs) {
  switch (d) {
    case 64: return mt_bs<T, 64>(bs);
    case 128: return mt_bs<T, 128>(bs);
  }
  return nullptr;
}

const void* multi_token_kernel_for(int dtype, int head_dim, int block_size) {
  switch (dtype) {
    case 0: return mt_d<float>(head_dim, block_size);
    case 1: return mt_d<_Float16>(head_dim, block_size);
    case 2: return mt_d<__bf16>(head_dim, block_size);
  }
  return nullptr;
}

template <typename T>
const void* merge_d(int d) {
  switch (d) {
    case 64: return (const void*)multi_token_merge_kernel<T, 64>;
    case 128: return (const void*)multi_token_merge_kernel<T, 128>;
  }
  return nullptr;
}

const void* multi_token_merge_for(int dtype, int head_dim) {
  switch (dtype) {
    case 0: return merge_d<float>(head_dim);
    case 1: return merge_d<_Float16>(head_dim);
    case 2: return merge_d<__bf16>(head_dim);
  }
  return nullptr;
}

}  // namespace

int multi_token_rows_per_group() { return ROWS; }

hipError_t launch_multi_token_merge(int dtype, int head_dim, const MultiTokenParams& p,
                                    hipStream_t stream) {
  const void* k = multi_token_merge_for(dtype, head_dim);
  const int64_t grid = (int64_t)p.row_tiles * p.num_kv_heads * p.num_seqs;
  if (!k || grid <= 0 || grid > 0x7fffffff || p.parts < 2) return hipErrorInvalidValue;
  MultiTokenParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(THREADS), args, 0, stream);
}

hipError_t launch_multi_token(int dtype, int head_dim, int block_size, MultiTokenParams p,
                              hipStream_t stream) {
  const void* k = multi_token_kernel_for(dtype, head_dim, block_size);
  const int64_t groups = (int64_t)p.num_kv_heads * p.num_seqs;
  const int64_t per_xcd = (groups + XCDS - 1) / XCDS * p.row_tiles * p.parts;
  if (!k || groups <= 0 || p.row_tiles <= 0 || p.parts <= 0 || per_xcd * XCDS > 0x7fffffff)
    return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(k, dim3((unsigned)(per_xcd * XCDS)), dim3(THREADS), args, 0, stream);
}

}  // namespace pa
