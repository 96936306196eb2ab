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
// row r is new token r / G, query head r % G of the group.  Each wave holds two 16-row
// MFMA tiles, tiles w and w + 4 of the workgroup's eight, so that a workgroup with few
// rows still spreads them over its waves; tiles without rows are skipped.  The
// workgroup walks the sequence's tokens in 32-token chunks up to the last position its
// rows may see; each chunk's K and V are gathered through the block table once, by
// global -> LDS loads with no register staging, into one of four LDS buffers (three
// chunks in flight while one is computed; two buffers for fp32 at head size 128), and
// read there by all four waves.
//
// MFMA layouts (as in the decode kernel, rows of the problem on the N side):
//   logits^T = K (32 tokens x D) . Q^T (D x 16 rows), two 16-token tiles per chunk
//   taking tokens {8i..8i+3} and {8i+4..8i+7}, so lane (row c, quad i) ends up holding
//   tokens 8i..8i+7 of row c: exactly the B operand (P^T) of
//   O^T += V^T (16 dims x 32 tokens) . P^T (32 tokens x 16 rows).
// K is stored in LDS in that MFMA row order, V segment-major (see Shape), so every
// operand is one 16-byte LDS read per lane, free of bank conflicts.
//
// Masking.  Positions past the causal limit of a row are removed by select (-inf
// before the max, weight 0).  Positions at or past L may hold anything: their logits are
// masked, and their values are cleared in LDS before the weighted sum.
//
// Precision.  Products accumulate in fp32.  The softmax weights enter the second product
// as a hi + lo pair of the 16-bit input type (8 or 11 significant bits alone would show
// next to the output's own rounding: a weight's rounding error reaches the output at
// the scale of the values, while averaging can make the output much smaller), and
// exactly for fp32; the sum that normalises them is kept in fp32.  Each row's exponent
// base moves only when a logit exceeds it by more than kLazyRescale, so weights lie in
// [0, 2^8] rather than [0, 1]: the same relative precision, and most chunks skip the
// rescale of the accumulators (FlashAttention-4's conditional rescaling).
//
// Context split.  With few (row tile, KV head, sequence) triples, as when a few draft
// tokens per sequence are verified against long contexts, the tokens of each sequence
// are cut into partitions of part_tokens positions, one workgroup each; every
// workgroup leaves its rows' exponent base, sum and unnormalised output in a
// workspace, and a second launch combines them with log-sum-exp weights.
//
// Launch.  One workgroup per (row tile, partition, KV head, sequence).  Workgroups are
// dispatched to the eight XCDs in turn; the numbering deals whole (sequence, KV head) groups to
// the XCDs round-robin, so that the row tiles of a group share their XCD's L2 copy of
// the K/V they all read, and every XCD gets a share of every sequence.
#include <float.h>
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
// Lazy rescaling (log2 units): the exponent base of a row moves only when a logit
// exceeds it by more than this, so weights stay below 2^8 and most chunks skip the
// rescale of the accumulators
constexpr float kLazyRescale = 8.f;

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

// Lazy rescaling of one row tile for one chunk.  lm is this lane's largest logit of the
// chunk in log2 units (the four lanes of a row share the row's base).  Only when some
// row of the wave has a logit above its base + kLazyRescale is the row maximum formed;
// such a row's base moves to it and what the row summed so far shrinks by
// exp2(old - new), while the other rows get exp2(0) = 1.
template <int NT>
__device__ __forceinline__ void rebase(float lm, float& m_base, float& l_run, f32x4 (&acc)[NT]) {
  if (__any(lm > m_base + kLazyRescale)) {
    const float cm = max_over_quads(lm);
    const float mb = cm > m_base + kLazyRescale ? cm : m_base;
    const float alpha = exp2_fast(m_base - mb);
    l_run *= alpha;
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) acc[nn] *= alpha;
    m_base = mb;
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// eight weights as MFMA operands of a 16-bit type: hi = nearest T, lo = nearest T to
// the remainder, converted two at a time
template <typename T>
__device__ __forceinline__ void split_weights(const float (&p)[8], u32x4& hi, u32x4& lo) {
  typedef typename std::conditional<std::is_same<T, __bf16>::value, bf16x2, f16x2>::type T2;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const T2 h = __builtin_convertvector((f32x2){p[2 * k], p[2 * k + 1]}, T2);
    hi[k] = __builtin_bit_cast(uint32_t, h);
    f32x2 w;  // hi, widened exactly
    if constexpr (std::is_same<T, __bf16>::value) {
      // a bf16 is the upper half of an fp32
      w = f32x2{__uint_as_float(hi[k] << 16), __uint_as_float(hi[k] & 0xFFFF0000u)};
    } else {
      w = __builtin_convertvector(h, f32x2);
    }
    const T2 l = __builtin_convertvector((f32x2){p[2 * k] - w[0], p[2 * k + 1] - w[1]}, T2);
    lo[k] = __builtin_bit_cast(uint32_t, l);
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

// LDS layout of one chunk (no padding; the bank spread comes from the layouts):
//   keys    [32 rows][KSEG segments of 16 bytes], rows in MFMA order, and segment j of
//           row r stored at position j ^ kswz(r): the 16 rows one MFMA operand read
//           touches then fall on 16 different 16-byte bank groups
//   values  [CH / TPS segments][D dimensions][TPS tokens]: a value operand read (one
//           segment, 16 consecutive dimensions) covers 256 consecutive bytes
// Both are filled by global -> LDS loads that put lane l's bytes at base + l * size;
// each lane picks the global address whose bytes belong at its slot.
template <typename T, int D, int BS>
struct Shape {
  static constexpr int E = sizeof(T);
  static constexpr int EPL = 16 / E;                 // elements per 16 bytes
  static constexpr int KL = D * E / 64;              // 16-byte operand reads per key row
  static constexpr int NT = D / 16;                  // 16-dimension output tiles
  static constexpr int KSEG = D * E / 16;            // 16-byte segments of a key row
  static constexpr int KI = CH * KSEG / 64 / WAVES;  // key loads per wave per chunk
  // the rows under one key load (64 / KSEG of them) are one run of 4 consecutive
  // tokens, except at KSEG = 8: two runs 8 tokens apart, in two blocks when BS <= 8
  static constexpr int NBK = (KSEG == 8 && BS <= 8) ? 2 : 1;
  static constexpr int TPS = 16 / E;                 // tokens per value segment
  static constexpr int VB = TPS <= BS ? 16 : 4;      // bytes per lane of a value load
  static constexpr int VI = CH * D * E / (64 * VB) / WAVES;  // value loads per wave per chunk
  static constexpr int NBV = VB == 16 ? 1 : 2;       // blocks under one value load
  static constexpr int CHUNK = CH * D;               // elements of K (and of V) per chunk
  static constexpr int NBUF = 2 * CHUNK * E <= 16384 ? 4 : 2;  // chunk buffers in LDS
  static constexpr int LOADS = KI + VI;              // loads per wave per chunk
  static_assert(KI >= 1 && VI >= 1, "chunk loads must cover the workgroup");
  static_assert(KSEG == 8 || KSEG == 16 || KSEG == 32, "key rows of 128, 256 or 512 bytes");
  static_assert(D % 64 == 0, "a value load covers one segment of 64 dimensions or more");
};

// rows of the LDS key tile are in MFMA order: token t = 8a + 4q + b sits at 16q + 4a + b
__device__ __forceinline__ constexpr int krow_of(int t) {
  return 16 * ((t >> 2) & 1) + 4 * (t >> 3) + (t & 3);
}
__device__ __forceinline__ constexpr int tok_of_krow(int r) {
  return 8 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3);
}
// segment swizzle of key row r: a different 16-byte bank group for each of 16 rows
template <int KSEG>
__device__ __forceinline__ constexpr int kswz(int r) {
  return KSEG >= 16 ? (r & 15) : ((r >> 1) & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// One global -> LDS load: lane l's SIZE bytes at g land at lds + l * SIZE.  Issued as
// inline assembly so that the compiler's wait insertion, which cannot tell the chunk
// buffers apart, does not wait for every load in flight before each LDS read; the waits
// for these loads are the pipeline's own (wait_loads_and_sync).
// Each statement sets M0 (the LDS destination) itself and lists it as clobbered.  The
// compiler warns that it cannot save a reserved register around such a statement; it
// never has to, because nothing else in the library's code reads or writes M0: every
// build disassembles the code objects and fails if any instruction other than these
// set-up + load sequences touches M0 (codecheck.py).
// With NTL the load is non-temporal: for K/V that no other workgroup reads.
template <int SIZE, bool NTL>
__device__ __forceinline__ void load_to_lds(const void* g, const void* lds) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)lds;
  if constexpr (SIZE == 16 && NTL) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 ::"s"(m), "v"(g) : "memory", "m0");
  } else if constexpr (SIZE == 16) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 ::"s"(m), "v"(g) : "memory", "m0");
  } else if constexpr (NTL) {
    static_assert(SIZE == 4, "16- or 4-byte loads");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt"
                 ::"s"(m), "v"(g) : "memory", "m0");
  } else {
    static_assert(SIZE == 4, "16- or 4-byte loads");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 ::"s"(m), "v"(g) : "memory", "m0");
  }
}

// Waits of the chunk pipeline.  The loads into LDS are counted by vmcnt; a wave waits
// until at most N of its own are outstanding, then the workgroup barrier makes every
// wave's data visible.  The barrier is issued directly (not through a release fence,
// which would also wait for the chunks still in flight); the LDS reads before it have
// returned (lgkmcnt(0)), so nothing of the buffer about to be refilled is still read.
template <int N>
__device__ __forceinline__ void wait_loads_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ONE_TILE: every (sequence, KV head) has one row tile (at most 128 rows, e.g. draft
// tokens).  Then every K/V byte is read by one workgroup, so the staging loads are
// non-temporal, and a wave skips a tile that holds no row of the problem.  Otherwise
// several row tiles share each chunk through L2 (prompt chunks): the staging loads keep
// the default policy, and a wave with any row computes both of its tiles (a tile with
// no row repeats a live row and is never stored).  With no per-tile branch the 16-bit
// chunk body needs few enough registers (168) for three workgroups a CU, whose waves
// overlap one another's MFMA and VALU work on each SIMD.
template <typename T, int D, int BS, bool ONE_TILE>
__global__ __launch_bounds__(THREADS, sizeof(T) == 2 ? (ONE_TILE ? 2 : 3) : 1) void multi_token_kernel(MultiTokenParams P) {
  typedef Shape<T, D, BS> SH;
  constexpr int KL = SH::KL, NT = SH::NT, EPL = SH::EPL, KSEG = SH::KSEG, TPS = SH::TPS;
  // three workgroups a CU for the all-tiles 16-bit instance: three chunk buffers
  constexpr int NBUF = (!ONE_TILE && sizeof(T) == 2 && SH::NBUF == 4) ? 3 : SH::NBUF;

  __shared__ __attribute__((aligned(16))) T sk[NBUF][SH::CHUNK];
  __shared__ __attribute__((aligned(16))) T sv[NBUF][SH::CHUNK];

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
  // the sequence's query range and length, read together (one round trip, not two):
  // the empty asm keeps the length's load ahead of the early returns, below which the
  // compiler would otherwise sink it
  const int q0 = P.query_start[s], q1 = P.query_start[s + 1];
  const int L = P.seq_lens[s];
  asm volatile("" ::"s"(L));
  const int n = q1 - q0;
  // rows that cannot be placed inside out[0 .. T) are never written
  if (q0 < 0 || n < 0 || q1 > P.num_tokens) return;
  const int nrows = n * G;
  const int R0 = x * ROWS;
  if (R0 >= nrows) return;
  const int rend = min(nrows, R0 + ROWS);

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
  // (a zero scale is taken as FLT_MIN: the same weights, all exactly 1, but a masked
  // logit of -inf then stays -inf after scaling instead of becoming NaN)
  const float sc = fabsf(P.scale_log2) == 0.f ? FLT_MIN : fabsf(P.scale_log2);
  const uint32_t qsign = P.scale_log2 < 0.f ? (sizeof(T) == 2 ? 0x80008000u : 0x80000000u) : 0u;
  // Row tile t of wave w holds rows 16 (w + 4t) .. 16 (w + 4t) + 15 of the workgroup's
  // 128, so that a workgroup with few rows (a few new tokens) spreads them over its
  // waves; a tile with no row of the problem is skipped (nlive: live tiles of the wave).
  const int nlive = (R0 + 16 * wave < rend) + (R0 + 16 * (wave + WAVES) < rend);
  u32x4 qf[NTILE][KL];
  int lim[NTILE];
  bool rvalid[NTILE];
  int64_t orow[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int rr = R0 + 16 * (wave + WAVES * t) + col;
    rvalid[t] = rr < rend;
    const int rc = min(rr, rend - 1);
    const int j = rc / G;
    lim[t] = ctx + j;
    orow[t] = (int64_t)(q0 + j) * Hq + g * G + rc % G;
    const T* qp = (const T*)P.q + orow[t] * D + quad * EPL;
    // a row past the tile repeats the tile's last row (so every load is in bounds and
    // they all go out together); its results are never stored
#pragma unroll
    for (int c = 0; c < KL; ++c) qf[t][c] = *reinterpret_cast<const u32x4*>(qp + c * 4 * EPL) ^ qsign;
  }

  // ---- chunk loading, global -> LDS.  Key load i of a wave fills 64 consecutive key
  // slots (16 bytes each), value load i 64 consecutive value slots (VB bytes each); the
  // tokens under one load lie in at most two blocks, whose ids are scalar table reads.
  // The lane's offset inside its block is the same for every chunk (chunks start on
  // block edges), so it is computed once.
  const int32_t AS4* tbls = (const int32_t AS4*)tbl;
  int bad = 0;
  int koff[SH::KI], voff[SH::VI];
  int kjr[SH::KI][SH::NBK], vjr[SH::VI][SH::NBV];  // blocks (within the chunk), uniform
#pragma unroll
  for (int i = 0; i < SH::KI; ++i) {
    const int I = wave + WAVES * i;
    const int p = 64 * I + lane;
    const int r = p / KSEG;
    const int t = tok_of_krow(r);
    koff[i] = (t % BS) * D + ((p % KSEG) ^ kswz<KSEG>(r)) * EPL;
#pragma unroll
    for (int u = 0; u < SH::NBK; ++u) kjr[i][u] = tok_of_krow(64 * I / KSEG + 4 * u) / BS;
  }
#pragma unroll
  for (int i = 0; i < SH::VI; ++i) {
    const int I = wave + WAVES * i;
    if constexpr (SH::VB == 16) {  // slot p: segment p / D, dimension p % D
      const int p = 64 * I + lane;
      voff[i] = (p % D) * BS + ((p / D) * TPS) % BS;
      vjr[i][0] = ((64 * I / D) * TPS) / BS;
    } else {  // 4-byte slots at block size 4: tokens 8s + 2w, 8s + 2w + 1 of segment s
      const int q = 64 * I + lane;
      const int w = q % 4;
      voff[i] = ((q / 4) % D) * BS + 2 * (w & 1);
#pragma unroll
      for (int u = 0; u < SH::NBV; ++u) vjr[i][u] = 2 * ((16 * I) / D) + u;
    }
  }
  auto block_id = [&](int j) { return tbls[min(j, last_blk)]; };
  auto checked = [&](int id) {  // ids outside the pool -> 0, and the workgroup's rows NaN
    const bool ok = (uint32_t)id < nblk32;
    bad |= !ok;
    return ok ? id : 0;
  };
  // table reads go out one chunk before their ids are used, and are checked only then
  int kid[SH::KI][SH::NBK], vid[SH::VI][SH::NBV];
  auto load_ids = [&](int c) {
    const int j0 = c * (CH / BS);
#pragma unroll
    for (int i = 0; i < SH::KI; ++i)
#pragma unroll
      for (int u = 0; u < SH::NBK; ++u) kid[i][u] = block_id(j0 + kjr[i][u]);
#pragma unroll
    for (int i = 0; i < SH::VI; ++i)
#pragma unroll
      for (int u = 0; u < SH::NBV; ++u) vid[i][u] = block_id(j0 + vjr[i][u]);
  };
  auto issue = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SH::KI; ++i) {
      int id = checked(kid[i][0]);
      if constexpr (SH::NBK == 2) {
        const int id1 = checked(kid[i][1]);
        id = lane >= 32 ? id1 : id;
      }
      load_to_lds<16, ONE_TILE>(kbase + (int64_t)id * blk_stride + koff[i],
                      &sk[buf][64 * (wave + WAVES * i) * EPL]);
    }
#pragma unroll
    for (int i = 0; i < SH::VI; ++i) {
      int id = checked(vid[i][0]);
      if constexpr (SH::NBV == 2) {
        const int id1 = checked(vid[i][1]);
        id = (lane & 2) ? id1 : id;
      }
      load_to_lds<SH::VB, ONE_TILE>(vbase + (int64_t)id * blk_stride + voff[i],
                          &sv[buf][64 * (wave + WAVES * i) * SH::VB / SH::E]);
    }
  };

  // per row: the exponent base and the running sum of the weights against it.  Until
  // the row sees a position the base is -FLT_MAX: the first finite logit moves it (its
  // rescale factor exp2(-FLT_MAX - m) is 0), and masked logits still give exp2(-inf) = 0
  float m_base[NTILE], l_run[NTILE];
  f32x4 acc[NTILE][NT];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    m_base[t] = -FLT_MAX;
    l_run[t] = 0.f;
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) acc[t][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One chunk: logits for both row tiles (the key operand read once for both), then per
  // tile the softmax and the weighted sum.  Only a chunk that crosses the causal limit of
  // some row of the workgroup is masked.
  auto compute = [&](int c, int buf) {
    if (nlive == 0) return;
    const int t0 = c * CH;
    const bool masked = t0 + CH - 1 > lim_lo;  // uniform
    // logits^T tiles a (tokens 8i..8i+3) and b (8i+4..8i+7); A read once for both row tiles
    f32x4 sa[NTILE], sb[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) sa[t] = sb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // every tile of a live wave (see ONE_TILE); fp32 keeps the per-tile order below
    constexpr bool ALL = !ONE_TILE && sizeof(T) == 2;
    // key rows col (tile a) and 16 + col (tile b) share their swizzle
    const T* ka = &sk[buf][col * KSEG * EPL];
    const T* kb = ka + 16 * KSEG * EPL;
    if constexpr (ALL) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int seg = (4 * k + quad) ^ kswz<KSEG>(col);
      const u32x4 a = *reinterpret_cast<const u32x4*>(ka + seg * EPL);
      const u32x4 b = *reinterpret_cast<const u32x4*>(kb + seg * EPL);
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        if (!ALL && t >= nlive) break;
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
    if constexpr (ALL) __builtin_amdgcn_s_setprio(0);
    // per row tile: softmax of the chunk, then its weighted sum
    const int tfirst = t0 + 8 * quad;
    // dimension 16nn + col, tokens 8quad .. 8quad + 7: value segment quad (two for fp32)
    const T* vrow = &sv[buf][(8 / TPS) * quad * D * TPS + col * TPS];
    if constexpr (ALL) {
      // Both tiles; masking first, on the logits (a masked logit is -inf, so its
      // weight is exp2(-inf) = 0 with no second select); then both softmaxes, then both
      // weighted sums.  Per tile the operations and their order are those of the loop
      // below, so the results are the same bits.  The waves raise their priority while
      // they issue MFMAs, so that a wave with matrix work ready issues it ahead of
      // another wave's vector work (measured 1% faster on chunked prefill).
      typedef typename V8<T>::type VT;
      static_assert(NTILE == 2, "two row tiles a wave");
      if (masked) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sa[t][e] = (tfirst + e <= lim[t]) ? sa[t][e] : -INFINITY;
            sb[t][e] = (tfirst + 4 + e <= lim[t]) ? sb[t][e] : -INFINITY;
          }
      }
      auto softmax = [&](int t, u32x4& hi, u32x4& lo) {
        float z[8];  // raw dot products; the scale is applied inside the exponent
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[e] = sa[t][e];
          z[4 + e] = sb[t][e];
        }
        rebase(max8(z) * sc, m_base[t], l_run[t], acc[t]);
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = exp2_fast(__builtin_fmaf(z[e], sc, -m_base[t]));
        float psum = pr[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) psum += pr[e];
        l_run[t] += psum;
        split_weights<T>(pr, hi, lo);
      };
      auto weighted_sum = [&](int t, const u32x4& hi, const u32x4& lo) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const VT vv = *reinterpret_cast<const VT*>(vrow + 16 * nn * TPS);
          acc[t][nn] = mma16(vv, __builtin_bit_cast(VT, hi), acc[t][nn]);
          acc[t][nn] = mma16(vv, __builtin_bit_cast(VT, lo), acc[t][nn]);
        }
        __builtin_amdgcn_s_setprio(0);
      };
      u32x4 h0, l0, h1, l1;
      softmax(0, h0, l0);
      softmax(1, h1, l1);
      weighted_sum(0, h0, l0);
      // tile 1 reads the value operands again rather than keeping tile 0's live
      uint32_t vaddr = (uint32_t)(uintptr_t)(lds_void*)vrow;
      asm volatile("" : "+v"(vaddr));
      vrow = (const T*)(lds_void*)(uintptr_t)vaddr;
      weighted_sum(1, h1, l1);
      return;
    }
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      if (t >= nlive) break;
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
      // a row with every position of this chunk masked has maximum -inf here and keeps
      // its base (a partition that starts past a row's causal limit leaves it at -FLT_MAX)
      rebase(max8(z) * sc, m_base[t], l_run[t], acc[t]);
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = exp2_fast(__builtin_fmaf(z[e], sc, -m_base[t]));
      if (masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = (tfirst + e <= lim[t]) ? pr[e] : 0.f;
      }
      float psum = pr[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) psum += pr[e];
      l_run[t] += psum;
      if constexpr (sizeof(T) == 2) {
        // the weights go in as a hi + lo pair (two MFMAs), about fp32 accuracy, so that
        // the output's own rounding is the only visible error
        typedef typename V8<T>::type VT;
        u32x4 phi, plo;
        split_weights<T>(pr, phi, plo);
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const VT vv = *reinterpret_cast<const VT*>(vrow + 16 * nn * TPS);
          acc[t][nn] = mma16(vv, __builtin_bit_cast(VT, phi), acc[t][nn]);
          acc[t][nn] = mma16(vv, __builtin_bit_cast(VT, plo), acc[t][nn]);
        }
      } else {
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(vrow + 16 * nn * TPS);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(vrow + 16 * nn * TPS + D * TPS);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][nn] = mma4(lo[e], pr[e], acc[t][nn]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][nn] = mma4(hi[e], pr[4 + e], acc[t][nn]);
        }
      }
    }
  };

  // ---- the chunk pipeline over chunks c_lo .. nch-1: NBUF - 1 chunks in flight
  // ahead of the one computed.  Positions at or past L may hold anything: values there
  // are cleared in LDS before use (their weights are 0, but 0 * NaN is not); keys there
  // only reach logits that are masked by select.
  // the query fragments arrive before the first chunk loads go out (the compiler, not
  // seeing those loads, would otherwise wait for all of them at the first use of Q)
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int c = 0; c < KL; ++c) asm volatile("" ::"v"(qf[t][c]));
  load_ids(c_lo);
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) {
    if (c_lo + j < nch) {
      issue((c_lo + j) % NBUF);
      if (c_lo + j + 1 < nch) load_ids(c_lo + j + 1);
    }
  }
  for (int c = c_lo; c < nch; ++c) {
    const int buf = c % NBUF;
    const int ahead = min(NBUF - 2, nch - 1 - c);  // chunks issued after this one
    if constexpr (NBUF == 4) {
      if (ahead >= 2) wait_loads_and_sync<2 * SH::LOADS>();
      else if (ahead == 1) wait_loads_and_sync<SH::LOADS>();
      else wait_loads_and_sync<0>();
    } else if constexpr (NBUF == 3) {
      if (ahead >= 1) wait_loads_and_sync<SH::LOADS>();
      else wait_loads_and_sync<0>();
    } else {
      wait_loads_and_sync<0>();
    }
    const int t0 = c * CH;
    if (t0 + CH > L) {
      for (int i = tid; i < (t0 + CH - L) * D; i += THREADS) {
        const int tok = L - t0 + i / D;
        sv[buf][((tok / TPS) * D + i % D) * TPS + tok % TPS] = (T)0.f;
      }
      lds_sync();
    }
    if (c + NBUF - 1 < nch) {
      issue((c + NBUF - 1) % NBUF);  // the buffer computed last iteration
      if (c + NBUF < nch) load_ids(c + NBUF);
    }
    compute(c, buf);
  }
  bad = __syncthreads_or(bad);

  if (split) {
    // this partition's partial rows for the merge: exponent base (log2 units; -inf for a
    // row that saw no position), sum and unnormalised output; a bad table entry makes
    // them NaN
    const int64_t tile0 =
        ((((int64_t)s * P.num_kv_heads + g) * P.row_tiles + x) * P.parts + part) * P.part_rows;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const float l = sum_over_quads(l_run[t]);
      if (!rvalid[t]) continue;
      const int64_t r = tile0 + 16 * (wave + WAVES * t) + col;
      float* po = P.part_o + r * D + 4 * quad;
#pragma unroll
      for (int nn = 0; nn < NT; ++nn)
        *reinterpret_cast<f32x4*>(po + 16 * nn) = bad ? f32x4{nan, nan, nan, nan} : acc[t][nn];
      const float mb = m_base[t] == -FLT_MAX ? -INFINITY : m_base[t];
      if (quad == 0)
        *reinterpret_cast<f32x2*>(P.part_ml + 2 * r) = bad ? f32x2{nan, nan} : f32x2{mb, l};
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

// The merge after a split launch.  A workgroup combines MROWS rows of one (row tile,
// KV head, sequence), one thread per (row, 4 dimensions), over the row's partitions
// with log-sum-exp weights in partition order (a running maximum, as in the main
// kernel's chunk loop), and writes the output rows (NaN rows for
// a length the table cannot hold).  Partitions that start past the tile's last causal
// limit were skipped by the main kernel and are not read; the first partition always
// holds position 0, which every row sees.
template <int D>
struct Merge {
  static constexpr int MROWS = THREADS / (D / 4);  // rows per workgroup
};

template <typename T, int D>
__global__ __launch_bounds__(THREADS) void multi_token_merge_kernel(MultiTokenParams P) {
  constexpr int MROWS = Merge<D>::MROWS;
  const int slabs = (P.part_rows + MROWS - 1) / MROWS;
  const int slab = (int)(blockIdx.x % slabs);
  const int tile = (int)(blockIdx.x / slabs);
  const int x = tile % P.row_tiles;
  const int group = tile / P.row_tiles;
  const int g = group % P.num_kv_heads;
  const int s = group / P.num_kv_heads;
  const int G = P.group, Hq = P.num_q_heads;
  const int q0 = P.query_start[s], q1 = P.query_start[s + 1];
  const int L = P.seq_lens[s];  // read beside the query range: one round trip
  asm volatile("" ::"s"(L));    // (kept ahead of the early return)
  const int n = q1 - q0;
  if (q0 < 0 || n < 0 || q1 > P.num_tokens) return;
  const int R0 = x * ROWS;
  const int rend = min(n * G, R0 + ROWS);
  const int r = slab * MROWS + (int)threadIdx.x / (D / 4);  // row within the tile
  if (R0 + r >= rend) return;
  const int d4 = ((int)threadIdx.x % (D / 4)) * 4;
  const int rr = R0 + r;
  T* o = (T*)P.out + ((int64_t)(q0 + rr / G) * Hq + g * G + rr % G) * D + d4;
  const float nan = __builtin_nanf("");
  if (L > P.max_tokens || n > L) {
    store4(o, f32x4{nan, nan, nan, nan});
    return;
  }
  const int lim_hi = L - n + (rend - 1) / G;
  const int used = min(P.parts, (lim_hi / CH) / (P.part_tokens / CH) + 1);
  const int64_t row0 = (((int64_t)s * P.num_kv_heads + g) * P.row_tiles + x) * P.parts * P.part_rows + r;
  const float* ml = P.part_ml + 2 * row0;
  const float* po = P.part_o + row0 * D + d4;
  const int64_t ps = P.part_rows;  // rows between one partition and the next
  // one pass in partition order with a running maximum: the loads of later partitions
  // do not wait for the arithmetic of earlier ones.  Partition 0 holds position 0, so
  // the maximum is finite from the first step on; a later partition none of whose
  // positions the row sees has maximum -inf and weight exp2(-inf) = 0.
  f32x2 v = *reinterpret_cast<const f32x2*>(ml);
  float M = v[0], Ls = v[1];
  f32x4 O = *reinterpret_cast<const f32x4*>(po);
  bool nan_seen = M != M;
#pragma unroll 8
  for (int p = 1; p < used; ++p) {
    v = *reinterpret_cast<const f32x2*>(ml + 2 * ps * p);
    const f32x4 op = *reinterpret_cast<const f32x4*>(po + ps * D * p);
    nan_seen |= v[0] != v[0];
    const float Mn = fmaxf(M, v[0]);
    const float a = exp2_fast(M - Mn), w = exp2_fast(v[0] - Mn);
    Ls = Ls * a + v[1] * w;
    O = O * a + op * w;
    M = Mn;
  }
  store4(o, nan_seen ? f32x4{nan, nan, nan, nan} : O / Ls);
}

template <typename T, int D, int BS>
const void* mt_nt(bool nt) {
  return nt ? (const void*)multi_token_kernel<T, D, BS, true>
            : (const void*)multi_token_kernel<T, D, BS, false>;
}

template <typename T, int D>
const void* mt_bs(int bs, bool nt) {
  switch (bs) {
    case 4: return mt_nt<T, D, 4>(nt);
    case 8: return mt_nt<T, D, 8>(nt);
    case 16: return mt_nt<T, D, 16>(nt);
    case 32: return mt_nt<T, D, 32>(nt);
  }
  return nullptr;
}

template <typename T>
const void* mt_d(int d, int bs, bool nt) {
  switch (d) {
    case 64: return mt_bs<T, 64>(bs, nt);
    case 128: return mt_bs<T, 128>(bs, nt);
  }
  return nullptr;
}

const void* multi_token_kernel_for(int dtype, int head_dim, int block_size, bool nt) {
  switch (dtype) {
    case 0: return mt_d<float>(head_dim, block_size, nt);
    case 1: return mt_d<_Float16>(head_dim, block_size, nt);
    case 2: return mt_d<__bf16>(head_dim, block_size, nt);
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
  const int mrows = head_dim == 64 ? Merge<64>::MROWS : Merge<128>::MROWS;
  const int64_t grid = (int64_t)p.row_tiles * p.num_kv_heads * p.num_seqs *
                       ((p.part_rows + mrows - 1) / mrows);
  if (!k || grid <= 0 || grid > 0x7fffffff || p.parts < 2) return hipErrorInvalidValue;
  MultiTokenParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(THREADS), args, 0, stream);
}

hipError_t launch_multi_token(int dtype, int head_dim, int block_size, MultiTokenParams p,
                              hipStream_t stream) {
  const void* k = multi_token_kernel_for(dtype, head_dim, block_size, p.row_tiles == 1);
  const int64_t groups = (int64_t)p.num_kv_heads * p.num_seqs;
  const int64_t per_xcd = (groups + XCDS - 1) / XCDS * p.row_tiles * p.parts;
  if (!k || groups <= 0 || p.row_tiles <= 0 || p.parts <= 0 || per_xcd * XCDS > 0x7fffffff)
    return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(k, dim3((unsigned)(per_xcd * XCDS)), dim3(THREADS), args, 0, stream);
}

}  // namespace pa
