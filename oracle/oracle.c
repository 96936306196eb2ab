/*
 * oracle.c - plain fp64 CPU reference for paged decode attention and for the
 * KV-cache write.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the only thing the two have in
 * common is the storage convention of the cache, restated below.
 *
 * Pages cited (title, site):
 *   [AB]  "什么是分页注意力（PagedAttention）？"            aiboss88.com wiki
 *   [CY]  "深入解析 PagedAttention：vLLM 显存优化的核心魔法"   cygnushan.xyz blog
 *   [ASP] "PagedAttention"                                 awesome-system-papers
 *   [RK]  "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?"  news.rkmt.cn
 *
 * What is computed.  Paging changes how the KV cache is stored and addressed,
 * never the attention formula itself ([AB] 边界与常见误解, first point; [ASP]
 * 相关工作, the entry on "Attention Is All You Need").  So the decode result for
 * one query head is textbook scaled dot-product attention over the sequence's
 * tokens in logical order, with each token's K and V fetched through the
 * per-sequence block table (logical block index -> physical block, [ASP] 核心思想;
 * [RK] 块表).  The oracle does exactly that: gather the sequence's K and V into
 * contiguous fp64 arrays through the table, then run a two-pass softmax.
 *
 * Storage convention (the pages fix none; this is the library's definition):
 *   k_cache[N][Hkv][bs][D]   token-major inside a block (one row = D elements)
 *   v_cache[N][Hkv][D][bs]   dimension-major inside a block
 *   q, out  [S][Hq][D]
 *   block_tables[S][max_blocks_per_seq] int32, entries past the used blocks are
 *   ignored (the pages pad them with -1, [CY] 核心思想 / Block Table)
 *   seq_lens[S] int32; token t of sequence s lives in physical block
 *   block_tables[s][t / bs] at in-block offset t % bs ([RK] 分页注意力是如何工作的,
 *   blocks numbered from 0 as in its block table).
 *   Query head h reads KV head h / (Hq / Hkv) (consecutive grouping).
 *   A slot id is phys * bs + offset; a negative slot id means "no write".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

enum {
  OR_OK = 0,
  OR_BAD_ARG = 1,    /* shapes, dtype or pointers invalid                    */
  OR_BAD_LEN = 2,    /* a sequence length < 0 or > max_blocks_per_seq * bs   */
  OR_BAD_BLOCK = 3,  /* a used table entry outside [0, num_blocks)           */
  OR_BAD_SLOT = 4,   /* a slot id >= num_blocks * bs                          */
  OR_DUP_SLOT = 5,   /* two tokens name the same slot                         */
  OR_NOMEM = 6
};

/* ---- element decoding (exact: every fp16 / bf16 / fp32 value is a double) -- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, sizeof x);
  return (double)x;
}

static double load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == OR_F32) {
    float x;
    memcpy(&x, (const char*)base + idx * 4, 4);
    return (double)x;
  }
  uint16_t b;
  memcpy(&b, (const char*)base + idx * 2, 2);
  return dtype == OR_F16 ? half_bits_to_double(b) : bf16_bits_to_double(b);
}

/* exported so tests can pin the decoding against independent libraries */
void oracle_decode_elements(const void* src, int64_t n, int32_t dtype, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, i, dtype);
}

int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ---- decode ---------------------------------------------------------------- */

static int64_t kpos(int64_t blk, int g, int o, int d, int Hkv, int bs, int D) {
  return (((blk * Hkv + g) * bs) + o) * (int64_t)D + d; /* k_cache[blk][g][o][d] */
}
static int64_t vpos(int64_t blk, int g, int o, int d, int Hkv, int bs, int D) {
  return (((blk * Hkv + g) * D) + d) * (int64_t)bs + o; /* v_cache[blk][g][d][o] */
}

/*
 * out[s][h][:] = sum_t w_t V[t][:] / sum_t w_t,
 *   w_t = exp(z_t - max_u z_u),  z_t = scale * <q[s][h], K[t]>,  t = 0 .. L_s - 1
 * with K[t], V[t] gathered through the block table.  L_s = 0 gives out = 0.
 * Everything after the element decode is fp64; no blocking, no splitting, no
 * online rescaling.  Returns an OR_* code; on error nothing is written.
 */
int oracle_decode(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                  int32_t dtype, double scale, double* out) {
  const int S = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads, D = head_dim;
  const int bs = block_size, MB = max_blocks_per_seq;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return OR_BAD_ARG;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || MB < 0 || num_blocks < 0)
    return OR_BAD_ARG;
  if (Hq % Hkv != 0) return OR_BAD_ARG;
  if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return OR_BAD_ARG;
  const int G = Hq / Hkv;

  /* 1. validate every sequence before computing anything */
  for (int s = 0; s < S; ++s) {
    const int L = seq_lens[s];
    if (L < 0 || (int64_t)L > (int64_t)MB * bs) return OR_BAD_LEN;
    const int nb = (L + bs - 1) / bs; /* blocks actually used */
    for (int j = 0; j < nb; ++j) {
      const int32_t b = block_tables[(int64_t)s * MB + j];
      if (b < 0 || (int64_t)b >= num_blocks) return OR_BAD_BLOCK;
    }
  }

  int failed = 0;
  /* 2. one independent task per (sequence, KV head) */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < (int64_t)S * Hkv; ++task) {
    const int s = (int)(task / Hkv), g = (int)(task % Hkv);
    const int L = seq_lens[s];
    if (L == 0) {
      for (int h = g * G; h < (g + 1) * G; ++h)
        for (int d = 0; d < D; ++d) out[((int64_t)s * Hq + h) * D + d] = 0.0;
      continue;
    }
    double* K = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    if (!K || !V || !z) {
      free(K);
      free(V);
      free(z);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    /* assemble the contiguous K and V of this sequence through the table */
    for (int t = 0; t < L; ++t) {
      const int64_t blk = block_tables[(int64_t)s * MB + t / bs];
      const int o = t % bs;
      for (int d = 0; d < D; ++d) {
        K[(int64_t)t * D + d] = load_elem(k_cache, kpos(blk, g, o, d, Hkv, bs, D), dtype);
        V[(int64_t)t * D + d] = load_elem(v_cache, vpos(blk, g, o, d, Hkv, bs, D), dtype);
      }
    }
    for (int h = g * G; h < (g + 1) * G; ++h) {
      const int64_t qo = ((int64_t)s * Hq + h) * D;
      /* logits */
      for (int t = 0; t < L; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += load_elem(q, qo + d, dtype) * K[(int64_t)t * D + d];
        z[t] = scale * acc;
      }
      /* numerically stable softmax: subtract the maximum, exponentiate, normalise */
      double m = z[0];
      for (int t = 1; t < L; ++t)
        if (z[t] > m) m = z[t];
      double Z = 0.0;
      for (int t = 0; t < L; ++t) {
        z[t] = exp(z[t] - m);
        Z += z[t];
      }
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int t = 0; t < L; ++t) acc += z[t] * V[(int64_t)t * D + d];
        out[qo + d] = acc / Z;
      }
    }
    free(K);
    free(V);
    free(z);
  }
  return failed ? OR_NOMEM : OR_OK;
}

/* ---- cache write ------------------------------------------------------------- */

static int cmp_i64(const void* a, const void* b) {
  const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/*
 * Each new token's K and V go into the slot its slot id names: block
 * slot / bs, offset slot % bs ([RK] 分页注意力是如何工作的: a token fills the next
 * free position of the sequence's current block; [ASP] 核心思想: a new block
 * only every bs tokens).  A bit copy; tokens with a negative slot are skipped.
 * k, v are [T][Hkv][D].  elem_bytes is 2 or 4.  Everything is checked before
 * anything is written.
 */
int oracle_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, int32_t elem_bytes,
                       void* k_cache, void* v_cache) {
  const int T = num_tokens, Hkv = num_kv_heads, D = head_dim, bs = block_size;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return OR_BAD_ARG;
  if (T < 0 || Hkv <= 0 || D <= 0 || bs <= 0 || num_blocks < 0) return OR_BAD_ARG;
  if (elem_bytes != 2 && elem_bytes != 4) return OR_BAD_ARG;

  int64_t* used = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
  if (!used) return OR_NOMEM;
  int n = 0;
  for (int i = 0; i < T; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= num_blocks * (int64_t)bs) {
      free(used);
      return OR_BAD_SLOT;
    }
    used[n++] = slot;
  }
  qsort(used, (size_t)n, sizeof(int64_t), cmp_i64);
  for (int i = 1; i < n; ++i)
    if (used[i] == used[i - 1]) {
      free(used);
      return OR_DUP_SLOT;
    }
  free(used);

  char* kc = (char*)k_cache;
  char* vc = (char*)v_cache;
  const char* ks = (const char*)k;
  const char* vs = (const char*)v;
  for (int i = 0; i < T; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    const int64_t blk = slot / bs;
    const int o = (int)(slot % bs);
    for (int g = 0; g < Hkv; ++g)
      for (int d = 0; d < D; ++d) {
        const int64_t src = ((int64_t)i * Hkv + g) * D + d;
        memcpy(kc + kpos(blk, g, o, d, Hkv, bs, D) * elem_bytes, ks + src * elem_bytes,
               (size_t)elem_bytes);
        memcpy(vc + vpos(blk, g, o, d, Hkv, bs, D) * elem_bytes, vs + src * elem_bytes,
               (size_t)elem_bytes);
      }
  }
  return OR_OK;
}

/* ---- several new tokens per sequence ------------------------------------------ */

/*
 * Attention for a chunk of new tokens per sequence (a prompt chunk when a new
 * sequence joins a step, or draft tokens to verify): [ASP] 实现要点 (continuous
 * batching adds sequences every step) and 已知局限 (speculative decoding over the
 * paged cache).  The formula is still the scaled dot-product attention the cache
 * serves ([ASP] 引用本概念的论文, "Attention Is All You Need"), whose decoder lets a
 * token see itself and every earlier token, never a later one.
 *
 * Sequence s has L_s tokens in the cache (seq_lens), the last n_s of them new, with
 * n_s = query_start[s+1] - query_start[s]; its queries are rows query_start[s] ..
 * query_start[s+1]-1 of q and out ([T][Hq][D]).  New token j (0-based) sits at
 * position c_s + j, c_s = L_s - n_s, and attends to positions 0 .. c_s + j:
 *   out[query_start[s]+j][h][:] = sum_t w_t V[t][:] / sum_t w_t,  t = 0 .. c_s + j,
 *   w_t = exp(z_t - max_u z_u),  z_t = scale * <q[query_start[s]+j][h], K[t]>.
 * With n_s = 1 this is oracle_decode.  query_start[0] = 0, query_start[S] = T,
 * non-decreasing, n_s <= L_s.  Returns an OR_* code; on error nothing is written.
 */
int oracle_multi_token(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens,
                       const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                       int32_t dtype, double scale, double* out) {
  const int S = num_seqs, T = num_tokens, Hq = num_q_heads, Hkv = num_kv_heads, D = head_dim;
  const int bs = block_size, MB = max_blocks_per_seq;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start || !out)
    return OR_BAD_ARG;
  if (S < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || MB < 0 || num_blocks < 0)
    return OR_BAD_ARG;
  if (Hq % Hkv != 0) return OR_BAD_ARG;
  if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return OR_BAD_ARG;
  if (query_start[0] != 0 || query_start[S] != T) return OR_BAD_ARG;
  const int G = Hq / Hkv;

  for (int s = 0; s < S; ++s) {
    const int L = seq_lens[s];
    const int n = query_start[s + 1] - query_start[s];
    if (n < 0) return OR_BAD_ARG;
    if (L < 0 || (int64_t)L > (int64_t)MB * bs || n > L) return OR_BAD_LEN;
    const int nb = (L + bs - 1) / bs;
    for (int j = 0; j < nb; ++j) {
      const int32_t b = block_tables[(int64_t)s * MB + j];
      if (b < 0 || (int64_t)b >= num_blocks) return OR_BAD_BLOCK;
    }
  }

  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < (int64_t)S * Hkv; ++task) {
    const int s = (int)(task / Hkv), g = (int)(task % Hkv);
    const int L = seq_lens[s];
    const int n = query_start[s + 1] - query_start[s];
    if (n == 0) continue;
    const int c = L - n;
    double* K = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    if (!K || !V || !z) {
      free(K);
      free(V);
      free(z);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    for (int t = 0; t < L; ++t) {
      const int64_t blk = block_tables[(int64_t)s * MB + t / bs];
      const int o = t % bs;
      for (int d = 0; d < D; ++d) {
        K[(int64_t)t * D + d] = load_elem(k_cache, kpos(blk, g, o, d, Hkv, bs, D), dtype);
        V[(int64_t)t * D + d] = load_elem(v_cache, vpos(blk, g, o, d, Hkv, bs, D), dtype);
      }
    }
    for (int j = 0; j < n; ++j) {
      const int last = c + j; /* the newest position this token may see */
      for (int h = g * G; h < (g + 1) * G; ++h) {
        const int64_t qo = ((int64_t)(query_start[s] + j) * Hq + h) * D;
        for (int t = 0; t <= last; ++t) {
          double acc = 0.0;
          for (int d = 0; d < D; ++d) acc += load_elem(q, qo + d, dtype) * K[(int64_t)t * D + d];
          z[t] = scale * acc;
        }
        double m = z[0];
        for (int t = 1; t <= last; ++t)
          if (z[t] > m) m = z[t];
        double Z = 0.0;
        for (int t = 0; t <= last; ++t) {
          z[t] = exp(z[t] - m);
          Z += z[t];
        }
        for (int d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int t = 0; t <= last; ++t) acc += z[t] * V[(int64_t)t * D + d];
          out[qo + d] = acc / Z;
        }
      }
    }
    free(K);
    free(V);
    free(z);
  }
  return failed ? OR_NOMEM : OR_OK;
}
