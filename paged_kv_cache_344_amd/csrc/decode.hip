// decode.hip - gfx950 kernels behind pa_decode.
//
// Pages cited (title, site): [AB] "什么是分页注意力（PagedAttention）？" aiboss88.com;
// [ASP] "PagedAttention" awesome-system-papers; [RK] "什么是 LLM 中的分页注意力(Paged
// Attention)?它是如何工作的?" news.rkmt.cn.
//
// What runs.  One workgroup (4 waves) per (sequence s, KV head g, 16-query-head
// tile, partition p of the sequence's tokens).  The attention formula is the plain
// one ([AB] 边界与常见误解: paging does not change it); what paging changes is that
// every 32-token chunk looks its physical blocks up in the block table and
// gathers K and V from wherever they sit ([ASP] 实现要点, the kernel that takes a
// block table; [RK] 块表).  Inside a block the reads stay contiguous ([ASP] 核心思想).
//
// Matrix cores.  The G query heads of one KV head share every K/V byte, so the
// logits of a 32-token chunk are a (tokens x D) by (D x heads) product and the
// weighted sum is a (D x tokens) by (tokens x heads) product.  Both run on MFMA
// 16x16 tiles (16x16x32 for f16/bf16, 16x16x4 for f32) with heads on the N side,
// padded to 16.  Operand layouts were chosen so that no byte moves between lanes:
//   * QK: A = K rows (M = 16 tokens, K = head dim), B = q^T.  A lane's A operand is
//     a 16-byte slice of one key row, loaded straight from HBM.
//   * The two QK tiles of a chunk take tokens {8i..8i+3} and {8i+4..8i+7} of the
//     chunk, i = 0..3, so the C layout of the logits leaves lane (head c, quad i)
//     holding tokens 8i..8i+7 of head c - exactly the B operand (P^T) of the next
//     product.
//   * PV: A = V^T (M = 16 dims, K = 32 tokens), B = P^T.  The value cache is stored
//     dimension-major inside a block, so a lane's A operand (8 consecutive tokens
//     of one dimension) is again one 16-byte load.
//   * The output O^T (dims x heads) keeps head c in lane column c, the same lane
//     column that owns head c's running max and sum, so the online-softmax rescale
//     never crosses lanes.
// LDS is used only to merge the four waves' partial results at the end.
//
// Softmax.  Online: per chunk, new max m' = max(m, max z), rescale the running sum
// and output by 2^(m - m'), add 2^(z - m').  Logits are in base-2 units (scale
// pre-multiplied by log2 e), so each weight is one v_exp_f32.  Positions past the
// sequence end are removed by select (never by multiplying: the unused slots of
// the last block may hold anything, and 0 * NaN = NaN).
//
// Precision.  Inputs are exact in the MFMA; products accumulate in fp32.  The
// softmax weights enter the weighted sum as a bf16/f16 hi + lo pair (two MFMAs),
// which keeps them to about fp32 accuracy.
//
// Split-K.  A partition with p > 0 or a sequence with more than one partition
// writes (max, sum, unnormalised output) to the workspace; decode_merge_kernel
// combines them with log-sum-exp weights in partition order.  Sequences that fit
// in one partition are finished by their only workgroup.
#include <math.h>

#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define AS4 __attribute__((address_space(4)))  // constant address space: scalar loads

constexpr int NW = kWavesPerGroup;

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec8<_Float16> {
  typedef f16x8 type;
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

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

// Registers of one 32-token chunk for one lane (column c = lane % 16, quad i = lane / 16).
template <typename T, int D>
struct Chunk {
  static constexpr int E = sizeof(T);
  static constexpr int KL = D * E / 64;  // 16-byte loads per key row: a quarter of the row
  static constexpr int VL = E / 2;       // 16-byte loads per value tile: 8 tokens
  static constexpr int NT = D / 16;      // 16-dimension output tiles
  u32x4 ka[KL];                          // key row of token tau_a(c), MFMA tile a
  u32x4 kb[KL];                          // key row of token tau_a(c) + 4, tile b
  u32x4 v[NT][VL];                       // values of tokens 8i..8i+7, dimension 16n + c
};

// logits tile: acc[r][c] += sum_d K[row r][d] * q[head c][d]
template <typename T, int D>
__device__ __forceinline__ f32x4 qk_tile(const u32x4 (&k)[Chunk<T, D>::KL],
                                         const u32x4 (&q)[Chunk<T, D>::KL]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
    typedef typename Vec8<T>::type V8;
#pragma unroll
    for (int c = 0; c < Chunk<T, D>::KL; ++c)
      acc = mma16(__builtin_bit_cast(V8, k[c]), __builtin_bit_cast(V8, q[c]), acc);
  } else {
    // bit-cast whole vectors: a bit-cast of one vector element is not safe here
#pragma unroll
    for (int c = 0; c < Chunk<T, D>::KL; ++c) {
      const f32x4 kf = __builtin_bit_cast(f32x4, k[c]);
      const f32x4 qv = __builtin_bit_cast(f32x4, q[c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma4(kf[e], qv[e], acc);
    }
  }
  return acc;
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(NW * 64) void decode_partitions_kernel(DecodeParams P) {
  typedef Chunk<T, D> C;
  constexpr int IDS = 32 / BS;  // physical blocks a 32-token chunk spans
  constexpr int NT = C::NT;
  constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte load

  __shared__ float sm_o[NW][16][D + 4];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ int sm_bad[NW];

  const int p = blockIdx.x;
  const int g = blockIdx.y / P.head_tiles;
  const int ht = blockIdx.y - g * P.head_tiles;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int Hq = P.num_q_heads;
  const int hbase = g * P.group + ht * 16;    // first query head of this tile
  const int nh = min(16, P.group - ht * 16);  // query heads in this tile

  const int L = ((const int32_t AS4*)P.seq_lens)[s];
  if (L <= 0 || L > P.max_tokens) {
    // empty sequence -> zeros; a length the table cannot hold -> NaN rows
    if (p == 0) {
      const T fill = (T)(L == 0 ? 0.f : __builtin_nanf(""));
      T* o = (T*)P.out + ((int64_t)s * Hq + hbase) * D;
      for (int i = threadIdx.x; i < nh * D; i += NW * 64) o[i] = fill;
    }
    return;
  }
  const int t_begin = p * P.part_tokens;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + P.part_tokens);
  const int nparts = (L + P.part_tokens - 1) / P.part_tokens;
  const int nchunks = (t_end - t_begin + 31) >> 5;
  const int last_blk = (L - 1) / BS;  // last table entry the sequence uses

  // query fragment: lane (c, i) holds the same slice of q[head c] that it holds of
  // each key row
  const bool hvalid = col < nh;
  const T* qrow = (const T*)P.q + ((int64_t)s * Hq + hbase + (hvalid ? col : 0)) * D + quad * EPL;
  u32x4 qf[C::KL];
#pragma unroll
  for (int c = 0; c < C::KL; ++c)
    qf[c] = hvalid ? ld16(qrow + c * 4 * EPL) : u32x4{0u, 0u, 0u, 0u};

  const int64_t tile = (int64_t)BS * D;  // elements of one (block, KV head) tile
  const int64_t blk_stride = (int64_t)P.num_kv_heads * tile;
  const T* kbase = (const T*)P.k_cache + (int64_t)g * tile;
  const T* vbase = (const T*)P.v_cache + (int64_t)g * tile;
  const int32_t AS4* tbl = (const int32_t AS4*)(P.block_tables + (int64_t)s * P.max_blocks);

  // lane-constant positions inside a chunk
  const int ka = 8 * (col >> 2) + (col & 3);  // token of this lane's key row, tile a
  const int kofs_a = (ka % BS) * D + quad * EPL;
  const int kofs_b = ((ka + 4) % BS) * D + quad * EPL;
  const int ra = ka / BS, rb = (ka + 4) / BS;
  const int rv = (8 * quad) / BS;  // block of this lane's 8 value tokens (BS >= 8)
  const int vofs = (BS >= 8) ? col * BS + (8 * quad) % BS : col * BS;

  // table entries are int32, so a pool larger than INT32_MAX blocks accepts them all
  const uint32_t nblk32 = (uint32_t)min(P.num_blocks, (int64_t)0x7fffffff);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  int bad = 0;

  auto issue = [&](C& c, int t0) {
    int ids[IDS];
    const int j0 = t0 / BS;
    // entries past the sequence's last block are never read; their tokens are
    // masked, so the last block stands in for them
#pragma unroll
    for (int i = 0; i < IDS; ++i) ids[i] = tbl[min(j0 + i, last_blk)];
#pragma unroll
    for (int i = 0; i < IDS; ++i) {
      const bool ok = (uint32_t)ids[i] < nblk32;
      bad |= !ok;
      ids[i] = ok ? ids[i] : 0;
    }
    // per-lane choice among the chunk's (uniform) block ids
    int idlanes = 0;
    if constexpr (IDS > 2) {
#pragma unroll
      for (int i = 0; i < IDS; ++i) {
        const int sid = __builtin_amdgcn_readfirstlane(ids[i]);
        asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(idlanes) : "s"(sid), "i"(i));
      }
    }
    auto pick = [&](int r) {
      if constexpr (IDS == 1) return ids[0];
      else if constexpr (IDS == 2) return r ? ids[1] : ids[0];
      else return __builtin_amdgcn_ds_bpermute(r << 2, idlanes);
    };
    const T* pa = kbase + (int64_t)pick(ra) * blk_stride + kofs_a;
    const T* pb = kbase + (int64_t)pick(rb) * blk_stride + kofs_b;
#pragma unroll
    for (int k = 0; k < C::KL; ++k) {
      c.ka[k] = ld16(pa + k * 4 * EPL);
      c.kb[k] = ld16(pb + k * 4 * EPL);
    }
    if constexpr (BS >= 8) {
      const T* pv = vbase + (int64_t)pick(rv) * blk_stride + vofs;
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int u = 0; u < C::VL; ++u) c.v[n][u] = ld16(pv + n * 16 * BS + u * EPL);
    } else {  // BS == 4: the 8 tokens straddle two blocks
      const T* lo = vbase + (int64_t)pick(2 * quad) * blk_stride + vofs;
      const T* hi = vbase + (int64_t)pick(2 * quad + 1) * blk_stride + vofs;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if constexpr (sizeof(T) == 2) {
          const u32x2 a = ld8(lo + n * 16 * BS), b = ld8(hi + n * 16 * BS);
          c.v[n][0] = u32x4{a[0], a[1], b[0], b[1]};
        } else {
          c.v[n][0] = ld16(lo + n * 16 * BS);
          c.v[n][1] = ld16(hi + n * 16 * BS);
        }
      }
    }
  };

  auto compute = [&](C& c, int t0) {
    const f32x4 sa = qk_tile<T, D>(c.ka, qf);
    const f32x4 sb = qk_tile<T, D>(c.kb, qf);
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = sa[e] * P.scale_log2;      // token t0 + 8i + e
      z[4 + e] = sb[e] * P.scale_log2;  // token t0 + 8i + 4 + e
    }
    const int tfirst = t0 + 8 * quad;
    const bool tail = t0 + 32 > t_end;  // uniform: only the last chunk of a partition
    if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (tfirst + e < t_end) ? z[e] : -INFINITY;
    }
    float cm = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, z[e]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float m_new = fmaxf(m_run, cm);
    const float alpha = exp2_fast(m_run - m_new);
    float pr[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = exp2_fast(z[e] - m_new);
      psum += pr[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] *= alpha;

    if (tail) {  // values past the end may be NaN: zero them, never multiply them
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t keep = ((tfirst + 2 * w < t_end) ? 0x0000FFFFu : 0u) |
                                  ((tfirst + 2 * w + 1 < t_end) ? 0xFFFF0000u : 0u);
            c.v[n][0][w] &= keep;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            c.v[n][e >> 2][e & 3] = (tfirst + e < t_end) ? c.v[n][e >> 2][e & 3] : 0u;
        }
      }
    }
    if constexpr (sizeof(T) == 2) {
      // weights as hi + lo pairs of the input type: the sum of two products keeps
      // ~16 significant bits of each fp32 weight, so the weighted sum is as exact as
      // an fp32 one and the only rounding left is the final store
      typedef typename Vec8<T>::type V8;
      V8 phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const T h = (T)pr[e];
        phi[e] = h;
        plo[e] = (T)(pr[e] - (float)h);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const V8 vv = __builtin_bit_cast(V8, c.v[n][0]);
        acc[n] = mma16(vv, phi, acc[n]);
        acc[n] = mma16(vv, plo, acc[n]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const f32x4 lo = __builtin_bit_cast(f32x4, c.v[n][0]);
        const f32x4 hi = __builtin_bit_cast(f32x4, c.v[n][1]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[n] = mma4(lo[e], pr[e], acc[n]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[n] = mma4(hi[e], pr[4 + e], acc[n]);
      }
    }
  };

  // Software pipeline: the next chunk's 16 loads are issued before this chunk's
  // math, so they are in flight while it runs (the compiler's wait counts keep
  // them outstanding; the buffer copy at the end of an iteration is register
  // renaming the compiler turns into moves).
  int ck = wave;
  if (ck < nchunks) {
    C A;
    issue(A, t_begin + 32 * ck);
    while (ck + NW < nchunks) {
      C B;
      issue(B, t_begin + 32 * (ck + NW));
      compute(A, t_begin + 32 * ck);
      A = B;
      ck += NW;
    }
    compute(A, t_begin + 32 * ck);
  }

  // merge the four waves (fixed order) through LDS
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (quad == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_run;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(&sm_o[wave][col][16 * n + 4 * quad]) = acc[n];
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();

  int anybad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) anybad |= sm_bad[w];
  for (int it = threadIdx.x; it < nh * (D / 4); it += NW * 64) {
    const int hh = it / (D / 4);
    const int d4 = (it - hh * (D / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][hh]);
    float Ls = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][hh];
      if (mw == -INFINITY) continue;  // this wave had no chunk
      const float e = exp2_fast(mw - M);
      Ls += e * sm_l[w][hh];
      O += e * *reinterpret_cast<const f32x4*>(&sm_o[w][hh][d4]);
    }
    if (anybad) {
      const float nan = __builtin_nanf("");
      M = Ls = nan;
      O = f32x4{nan, nan, nan, nan};
    }
    const int64_t row = (int64_t)s * Hq + hbase + hh;
    if (nparts == 1) {
      T* o = (T*)P.out + row * D + d4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (T)(O[e] / Ls);
    } else {
      const int64_t slot = row * P.pmax + p;
      *reinterpret_cast<f32x4*>(P.ws_o + slot * D + d4) = O;
      if (d4 == 0) {
        P.ws_ml[2 * slot] = M;
        P.ws_ml[2 * slot + 1] = Ls;
      }
    }
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Log-sum-exp merge of a sequence's partitions, one workgroup per (query head,
// sequence).  Fixed reduction order, so the result does not depend on timing.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams P) {
  extern __shared__ float sm_w[];  // one weight per partition
  __shared__ float sm_red[4];
  __shared__ f32x4 sm_acc[256];
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = ((const int32_t AS4*)P.seq_lens)[s];
  if (L <= P.part_tokens || L > P.max_tokens) return;  // finished by its single partition
  const int nparts = (L + P.part_tokens - 1) / P.part_tokens;
  const int64_t row = (int64_t)s * P.num_q_heads + h;
  const float* ml = P.ws_ml + row * P.pmax * 2;
  const float* o = P.ws_o + row * P.pmax * D;

  float M = -INFINITY;
  for (int q = tid; q < nparts; q += 256) M = fmaxf(M, ml[2 * q]);
  M = wave_max(M);
  if (lane == 0) sm_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sm_red[0], sm_red[1]), fmaxf(sm_red[2], sm_red[3]));
  __syncthreads();

  float Ls = 0.f;
  for (int q = tid; q < nparts; q += 256) {
    const float w = exp2_fast(ml[2 * q] - M);
    sm_w[q] = w;
    Ls += w * ml[2 * q + 1];
  }
  Ls = wave_sum(Ls);
  if (lane == 0) sm_red[wave] = Ls;
  __syncthreads();
  Ls = (sm_red[0] + sm_red[1]) + (sm_red[2] + sm_red[3]);

  constexpr int C4 = D / 4;   // float4 columns of a row
  constexpr int R = 256 / C4; // rows summed in parallel
  const int r = tid / C4, c = tid - r * C4;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  for (int q = r; q < nparts; q += R)
    a += sm_w[q] * *reinterpret_cast<const f32x4*>(o + (int64_t)q * D + 4 * c);
  sm_acc[tid] = a;
  __syncthreads();
  if (tid < C4) {
    f32x4 t = sm_acc[tid];
#pragma unroll
    for (int rr = 1; rr < R; ++rr) t += sm_acc[rr * C4 + tid];
    T* out = (T*)P.out + row * D + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (T)(t[e] / Ls);
  }
}

template <typename T, int D, int BS>
hipError_t launch_parts(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.pmax, p.num_kv_heads * p.head_tiles, p.num_seqs);
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)decode_partitions_kernel<T, D, BS>, grid, dim3(NW * 64),
                         args, 0, stream);
}

template <typename T, int D>
hipError_t launch_parts_bs(int bs, const DecodeParams& p, hipStream_t stream) {
  switch (bs) {
    case 4: return launch_parts<T, D, 4>(p, stream);
    case 8: return launch_parts<T, D, 8>(p, stream);
    case 16: return launch_parts<T, D, 16>(p, stream);
    case 32: return launch_parts<T, D, 32>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_parts_d(int d, int bs, const DecodeParams& p, hipStream_t stream) {
  switch (d) {
    case 64: return launch_parts_bs<T, 64>(bs, p, stream);
    case 128: return launch_parts_bs<T, 128>(bs, p, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.num_q_heads, p.num_seqs);
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)decode_merge_kernel<T, D>, grid, dim3(256), args,
                         sizeof(float) * (size_t)p.pmax, stream);
}

template <typename T>
hipError_t launch_merge_d(int d, const DecodeParams& p, hipStream_t stream) {
  switch (d) {
    case 64: return launch_merge<T, 64>(p, stream);
    case 128: return launch_merge<T, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_partitions(int dtype, int head_dim, int block_size,
                                    const DecodeParams& p, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_parts_d<float>(head_dim, block_size, p, stream);
    case 1: return launch_parts_d<_Float16>(head_dim, block_size, p, stream);
    case 2: return launch_parts_d<__bf16>(head_dim, block_size, p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(int dtype, int head_dim, const DecodeParams& p,
                               hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_merge_d<float>(head_dim, p, stream);
    case 1: return launch_merge_d<_Float16>(head_dim, p, stream);
    case 2: return launch_merge_d<__bf16>(head_dim, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
