// decode.hip - the gfx950 kernel behind pa_decode.
//
// Pages cited (title, site): [AB] "什么是分页注意力（PagedAttention）？" aiboss88.com;
// [ASP] "PagedAttention" awesome-system-papers; [RK] "什么是 LLM 中的分页注意力(Paged
// Attention)?它是如何工作的?" news.rkmt.cn.
//
// What is computed.  For every sequence s and query head h, softmax attention of
// q[s][h] over the sequence's keys and values in logical order.  Paging leaves
// that formula alone ([AB] 边界与常见误解); what it changes is where token t lives:
// in physical block block_tables[s][t / bs] at offset t % bs ([RK] 块表), so the
// kernel looks each block up in the table and gathers it from wherever it sits
// ([ASP] 实现要点, the kernel that takes a block table).  Inside a block the reads
// are contiguous ([ASP] 核心思想).
//
// Work items.  A sequence is cut into partitions of part_tokens tokens (with the
// default size, as long as the load balance allows: see the plan); a work item is
// (sequence, partition, KV head, tile of up to 16 of its query heads) and is
// handled by one 4-wave workgroup.  The launch is persistent: about as many
// workgroups as fit on the chip at once, each taking items from a queue counter
// until none are left.  Lengths live in device memory, so every workgroup first
// plans for itself, in LDS, from seq_lens: it enumerates only the partitions that
// hold tokens (no workgroup is spent on partitions past a sequence's end), full
// partitions first and then each sequence's last, partly filled partition in
// decreasing size, so that the last items to start are the short ones.  Sequences of a
// single 32-token chunk come after those, four (sequence, head tile) items to a
// workgroup, one per wave, each wave finishing its own item without the LDS merge.
// Every workgroup computes the same plan.  A workgroup takes its next item when wave 0
// reaches its last chunk of the current one, so that items leave the queue in queue
// order rather than being held while other workgroups run dry.
//
// Inside an item the four waves take 32-token chunks in turn.  The G query heads of
// one KV head share every K/V byte, so the logits of a chunk are a (tokens x D) by
// (D x heads) product and the weighted sum is a (D x tokens) by (tokens x heads)
// product; both run on 16x16 MFMA tiles (16x16x32 for f16/bf16, 16x16x4 for f32)
// with the heads on the N side, padded to 16.  Operand layouts were chosen so that
// no byte moves between lanes:
//   * QK: A = K rows (M = 16 tokens, K = head dim), B = q^T.  A lane's A operand is a
//     16-byte slice of one key row, loaded straight from HBM.
//   * The two QK tiles of a chunk take tokens {8i..8i+3} and {8i+4..8i+7} of the chunk,
//     i = 0..3, so the C layout of the logits leaves lane (head c, quad i) holding
//     tokens 8i..8i+7 of head c: exactly the B operand (P^T) of the next product.
//   * PV: A = V^T (M = 16 dims, K = 32 tokens), B = P^T.  The value cache is stored
//     dimension-major inside a block, so a lane's A operand (8 consecutive tokens of
//     one dimension) is again one 16-byte load.
//   * The output O^T (dims x heads) keeps head c in lane column c, the lane column
//     that owns head c's running max and sum, so the softmax rescale never crosses
//     lanes.
// Each wave keeps two chunks' loads in flight (ping-pong register buffers).
//
// Softmax.  Online: per chunk, new max m' = max(m, max z), rescale the running sum
// and output by 2^(m - m'), add 2^(z - m').  Logits are in base-2 units (scale
// pre-multiplied by log2 e), so each weight is one v_exp_f32.  Positions past the
// sequence end are removed by select, never by multiplying: the unused slots of the
// last block may hold anything, and 0 * NaN = NaN.
//
// Precision.  Inputs are exact in the MFMA; products accumulate in fp32.  The
// softmax weights enter the weighted sum as a bf16/f16 hi + lo pair (two MFMAs),
// which keeps them to about fp32 accuracy.
//
// Cache policy.  With no block shared between tables, every K/V byte is read once per
// call and the loads are non-temporal (NTL); shared blocks keep the default policy so
// that they stay cached for the other sequences.
//
// Split-K merge.  A sequence with one partition is finished by its only item.
// Otherwise each item stores (max, sum, unnormalised output) per head; partitions
// form groups of 16, and the item that completes a group (an arrival counter)
// combines the group with log-sum-exp weights, and the item that completes the
// last group combines the groups.  The group arrival's answer is read at the
// workgroup's next item start, under that item's first loads.  The tree is fixed by
// partition numbers, so the result does not depend on timing or on which workgroup
// ran what.  Counters are reset by whoever finishes them, so they are all zero again
// after a call.
#include <math.h>

#include "decode_common.h"

namespace pa {
namespace {

using namespace dec;

constexpr int kWriteRows = 16;  // (token, KV head) rows a workgroup stores per claim (fused write)

// Diagnostic build only (PA_DECODE_TRACE, a separate library, never the product one):
// every workgroup records s_memrealtime stamps (100 MHz) of its plan and of its first
// kTraceItems items in kTraceWords words of pa_trace_buf: [0] entry, [1] plan done, [2 + 4k ..
// 5 + 4k] item k's start, end of its chunk loop, end of its epilogue and (queue position,
// one-chunk group flag << 32, past-the-regular-items flag << 33, tokens << 34), [248]
// lengths read,
// [250] partition length, [254] items taken, [255] exit.  Read back with
// pa_decode_trace_read; paged_kv_cache_344_amd/trace_decode.py prints the timeline.
#ifdef PA_DECODE_TRACE
constexpr int kTraceWords = 256;
constexpr int kTraceItems = 60;
__device__ unsigned long long pa_trace_buf[2048 * kTraceWords];
#define PA_TRACE_STAMP() __builtin_amdgcn_s_memrealtime()
#endif

// Log-sum-exp combination of cnt partials for each of nh heads.  Head hh's partials
// are slots (row0 + hh) * stride + first + i, i < cnt, of (src_o, src_ml); the result
// goes to the output rows (normalised, rounded) when out is given, else to slot
// (row0 + hh) * dstride + dslot of (dst_o, dst_ml).  Partials are combined in slot
// order, so the result is the same whoever runs it.
template <typename T, int D>
__device__ void merge_partials(const float* src_o, const float* src_ml, int64_t row0, int stride,
                               int first, int cnt, int nh, T* out, float* dst_o, float* dst_ml,
                               int dstride, int dslot, int Hq) {
  constexpr int C4 = D / 4;
  for (int it = threadIdx.x; it < nh * C4; it += NT_THREADS) {
    const int hh = it / C4, c = it - hh * C4;
    // partial slots are [sequence][partition][query head]
    const int64_t sq = row0 / Hq, h = row0 - sq * Hq + hh;
    const int64_t base = (sq * stride + first) * Hq + h;
    const float* ml = src_ml + 2 * base;
    // Loads go out in batches of 8 before any is used: device-scope loads keep
    // program order, so a use right after each load would wait on each one.
    float M = -INFINITY;
    for (int i0 = 0; i0 < cnt; i0 += 8) {
      float mv[8], lv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) ld_dev2(ml + 2 * (int64_t)min(i0 + k, cnt - 1) * Hq, mv[k], lv[k]);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (i0 + k < cnt) M = fmaxf(M, mv[k]);
    }
    float Ls = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < cnt; i0 += 8) {
      float mv[8], lv[8];
      f32x4 ov[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = min(i0 + k, cnt - 1);
        ld_dev2(ml + 2 * (int64_t)i * Hq, mv[k], lv[k]);
        ov[k] = ld_dev16(src_o + (sq * stride + first + i) * Hq * D, (int)((row0 - sq * Hq + hh) * D + 4 * c) * 4);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (i0 + k < cnt) {
          const float w = exp2_fast(mv[k] - M);
          Ls += w * lv[k];
          O += w * ov[k];
        }
      }
    }
    if (out) {
      store4(out + (row0 + hh) * D + 4 * c, O / Ls);
    } else {
      const int64_t d = (sq * dstride + dslot) * Hq + h;
      st_dev16(dst_o + (sq * dstride + dslot) * Hq * D, (int)((row0 - sq * Hq + hh) * D + 4 * c) * 4, O);
      if (c == 0) st_dev2(dst_ml + 2 * d, M, Ls);
    }
  }
}

// NTL: K and V are loaded non-temporally (no table shares a block, so every byte is
// read once per call); otherwise with the default policy, so that blocks several
// tables share stay in L2 and the Infinity Cache for the other sequences.
template <typename T, int D, int BS, bool NTL, bool FUSE>
__global__ __launch_bounds__(NT_THREADS, sizeof(T) == 2 ? 2 : 1) void decode_kernel(DecodeParams P) {
  typedef Chunk<T, D> C;
  constexpr int IDS = 32 / BS;  // physical blocks a 32-token chunk spans
  constexpr int NT = C::NT;
  constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte load

  __shared__ float sm_o[NW][16][D + 4];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ int sm_bad[NW];
  __shared__ int sm_len[kScanMax];       // seq_lens of the launch's sequences
  __shared__ int64_t sm_slot[FUSE ? kScanMax : 1];  // (fused write) slot_mapping of the sequences
  __shared__ int sm_full[kScanMax + 1];  // exclusive prefix count of full partitions
  __shared__ int sm_class[kScanMax];     // size class of each sequence's last partition
  __shared__ int sm_last[kScanMax];      // sequences in the order their last partitions run
  __shared__ int sm_ccount[kScanMax / 64][kSizeClasses];
  __shared__ int sm_ctotal[kSizeClasses];
  __shared__ int sm_cbase[kSizeClasses];
  __shared__ int sm_wsum[NW];
  __shared__ float sm_wsumf[NW];
  __shared__ int sm_wmax[NW], sm_wcnt[NW];
  __shared__ int sm_next[2];  // by item parity: an item may pass no barrier before the next write
  __shared__ int sm_flag[2];
#ifdef PA_DECODE_TRACE
  const unsigned long long tr_t0 = PA_TRACE_STAMP();
  unsigned long long* tr = pa_trace_buf + (blockIdx.x & 2047) * kTraceWords;
  int tr_n = 0;
#endif

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int S = P.num_seqs, Hq = P.num_q_heads;
  int PT = P.part_tokens;  // set by the plan when it chooses the partition size
  const int HT2 = P.num_kv_heads * P.head_tiles;


  // ---------------------------------------------------------------- plan
  // Thread t looks at sequences 4t .. 4t+3.  With the default partition size the
  // partition length is chosen first, from the lengths: every item ends with a merge
  // and, when split, partial results to write and merge later, which costs about as
  // much per item whatever its length, so partitions are made as long as the load
  // balance allows: kPartShare times one workgroup's even share of all the (token, KV
  // head tile) work, rounded up to a multiple of 256 tokens, never below part_tokens
  // (kTailShare of the share instead when at that length no sequence would be split
  // but there are more units than workgroups).
  // Every workgroup computes the same sum in the same order, so all choose alike.
  // Then: the number of full partitions of each sequence and the class of its last one
  // (0: an empty or invalid sequence, a one-item fill; 1: one chunk; 2 ..
  // kSizeClasses - 1 by the last partition's size).
  {
    int Ls[4];
    float lsum = 0.f;
    int lmax = 0, lcnt = 0;
    // every load first, from an index clamped into the launch's S >= 1 sequences, so
    // that all of them are in flight together: behind the per-sequence test below the
    // compiler issued them one at a time, each waiting for the one before
    int Lr[4];
    int64_t slot_r[4] = {};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sc = min(4 * tid + i, S - 1);
      Lr[i] = P.seq_lens[sc];
      if constexpr (FUSE) slot_r[i] = P.slot_mapping[sc];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * tid + i;
      Ls[i] = 0;
      if (s < S) {
        const int L = Lr[i];
        sm_len[s] = L;
        if constexpr (FUSE) sm_slot[s] = slot_r[i];
        if (L > 0 && L <= P.max_tokens) Ls[i] = L;
      }
      lsum += (float)Ls[i];
      lmax = max(lmax, Ls[i]);
      lcnt += Ls[i] > 0;
    }
    if (P.auto_part) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        lsum += __shfl_xor(lsum, o);
        lmax = max(lmax, __shfl_xor(lmax, o));
        lcnt += __shfl_xor(lcnt, o);
      }
      if (lane == 0) {
        sm_wsumf[wave] = lsum;
        sm_wmax[wave] = lmax;
        sm_wcnt[wave] = lcnt;
      }
      __syncthreads();
      float tot = 0.f;
      int mx = 0, cnt = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        tot += sm_wsumf[w];
        mx = max(mx, sm_wmax[w]);
        cnt += sm_wcnt[w];
      }
      const float share = tot * (float)HT2 / (float)gridDim.x;  // tokens per workgroup
      int pt = (int)ceilf(fminf(kPartShare * share, (float)P.max_tokens) * (1.f / 256.f)) * 256;
      // no sequence would be split, yet there are more (sequence, head tile) units than
      // workgroups: the longest units would set the tail, so split them after all
      if (pt >= mx && (int64_t)cnt * HT2 > (int64_t)gridDim.x)
        pt = (int)ceilf(fminf(kTailShare * share, (float)P.max_tokens) * (1.f / 256.f)) * 256;
      PT = max(PT, pt);
    }
#ifdef PA_DECODE_TRACE
    if (threadIdx.x == 0) tr[248] = PA_TRACE_STAMP();
#endif
    int nfull[4], cls[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int L = Ls[i];
      nfull[i] = cls[i] = 0;
      if (L > 0) {
        const int n = (L + PT - 1) / PT;
        const int r = L - (n - 1) * PT;  // tokens in the last partition, 1..PT
        nfull[i] = n - 1;
        cls[i] = L <= 32 ? 1
                         : 2 + (int)min((int64_t)(kSizeClasses - 3),
                                        ((int64_t)(r - 1) * (kSizeClasses - 2)) / PT);
      }
      sum += nfull[i];
    }
    const int incl = wave_incl_scan(sum, lane);
    if (lane == 63) sm_wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += sm_wsum[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * tid + i;
      if (s < S) {
        sm_full[s] = run;
        sm_class[s] = cls[i];
      }
      run += nfull[i];
    }
    if (tid == 0) {
      int F = 0;
      for (int w = 0; w < NW; ++w) F += sm_wsum[w];
      sm_full[S] = F;
    }
  }
  __syncthreads();
  PT = __builtin_amdgcn_readfirstlane(PT);
  // the partition length this launch uses, for the caller to read back (not a counter)
  if (blockIdx.x == 0 && tid == 0) P.queue[kPartSlot] = PT;
  // Stable counting sort of the sequences by size class, largest class first, and the
  // queue layout it gives: regular items (full partitions, then last partitions by
  // decreasing size), then one-chunk sequences NW items to a workgroup (one per wave),
  // then the fill items of empty or invalid sequences.
  const int F = sm_full[S];
  int c0 = 0, c1 = 0, jt0 = 0, A = 0, Gt = 0, total = 0;
  auto finish_plan = [&]() {
    const int ngroups = (S + 63) / 64;
    for (int j = wave; j < ngroups; j += NW) {
      const int s = 64 * j + lane;
      const int cls = s < S ? sm_class[s] : -1;
      int c = 0;
#pragma unroll
      for (int b = 0; b < kSizeClasses; ++b) {
        const int n = __popcll(__ballot(cls == b));
        if (lane == b) c = n;
      }
      if (lane < kSizeClasses) sm_ccount[j][lane] = c;
    }
    __syncthreads();
    if (tid < kSizeClasses) {
      int run = 0;
      for (int j = 0; j < ngroups; ++j) {
        const int c = sm_ccount[j][tid];
        sm_ccount[j][tid] = run;  // sequences of this class in earlier groups
        run += c;
      }
      sm_ctotal[tid] = run;
    }
    __syncthreads();
    if (tid < kSizeClasses) {
      int base = 0;
      for (int b = tid + 1; b < kSizeClasses; ++b) base += sm_ctotal[b];
      sm_cbase[tid] = base;
    }
    __syncthreads();
    for (int j = wave; j < ngroups; j += NW) {
      const int s = 64 * j + lane;
      const int cls = s < S ? sm_class[s] : -1;
      uint64_t same = 0;
#pragma unroll
      for (int b = 0; b < kSizeClasses; ++b) {
        const uint64_t m = __ballot(cls == b);
        if (cls == b) same = m;
      }
      if (s < S) {
        const int rank = __popcll(same & ((1ull << lane) - 1ull));
        sm_last[sm_cbase[cls] + sm_ccount[j][cls] + rank] = s;
      }
    }
    __syncthreads();
    c0 = sm_ctotal[0];
    c1 = sm_ctotal[1];
    jt0 = F + S - c0 - c1;            // first one-chunk entry
    A = jt0 * HT2;                    // regular items
    Gt = (c1 * HT2 + NW - 1) / NW;    // groups of one-chunk items
    total = A + Gt + c0 * HT2;        // the host keeps (F + S) * HT2 below 2^31
  };
  // A workgroup whose first item is a full partition (known from the scan alone) sorts
  // after issuing that item's first loads, so that the sort runs while they are in
  // flight; the others sort first.
  bool planned = false;
  if ((int64_t)blockIdx.x >= (int64_t)F * HT2) {
    finish_plan();
    planned = true;
  }

#ifdef PA_DECODE_TRACE
  if (threadIdx.x == 0) {
    tr[0] = tr_t0;
    tr[1] = PA_TRACE_STAMP();
    tr[250] = PT;
  }
#endif
  // table entries are int32, so a pool larger than INT32_MAX blocks accepts them all
  const uint32_t nblk32 = (uint32_t)min(P.num_blocks, (int64_t)0x7fffffff);
  const int64_t tile = (int64_t)BS * D;  // elements of one (block, KV head) tile
  const int64_t blk_stride = (int64_t)P.num_kv_heads * tile;

  // lane-constant positions inside a chunk
  const int ka = 8 * (col >> 2) + (col & 3);  // token of this lane's key row, tile a
  const int kofs_a = (ka % BS) * D + quad * EPL;
  const int kofs_b = ((ka + 4) % BS) * D + quad * EPL;
  const int ra = ka / BS, rb = (ka + 4) / BS;
  const int rv = (8 * quad) / BS;  // block of this lane's 8 value tokens (BS >= 8)
  const int vofs = (BS >= 8) ? col * BS + (8 * quad) % BS : col * BS;

  // ---------------------------------------------------------------- items
  // A split item's arrival in its merge group is issued at the end of the item, and its
  // answer (was this the group's last member?) is acted on when the workgroup next
  // settles: at the start of its next item, once that item's first loads have gone out,
  // or after the item loop.  The member that completed a group merges it there, under
  // those loads.  (The compiled loop carries the answer in a register copy that waits
  // for the atomic at the end of the item; measured, that wait is not on the critical
  // path, since the compute unit's other workgroup keeps streaming meanwhile.)
  bool pend = false;   // (uniform) an arrival whose answer has not been read
  int pend_before = 0;  // (thread 0) the arrival's answer: members counted before it
  int pend_s = 0, pend_gt = 0, pend_grp = 0, pend_gsize = 0, pend_ngrp = 0, pend_nh = 0,
      pend_n = 0;
  int64_t pend_row0 = 0;
  auto settle = [&]() {
    if (tid == 0) {
      const int done = pend_before == pend_gsize - 1;
      // every member has arrived: ready for the next call
      if (done) atomicExch(P.node_count + ((int64_t)pend_s * HT2 + pend_gt) * P.nodes + pend_grp, 0);
      sm_flag[0] = done;
    }
    __syncthreads();
    if (sm_flag[0]) {
      if (pend_ngrp == 1) {
        merge_partials<T, D>(P.part_o, P.part_ml, pend_row0, P.pmax, 0, pend_n, pend_nh,
                             (T*)P.out, nullptr, nullptr, 0, 0, Hq);
      } else {
        merge_partials<T, D>(P.part_o, P.part_ml, pend_row0, P.pmax, pend_grp * kMergeFan,
                             pend_gsize, pend_nh, (T*)nullptr, P.node_o, P.node_ml, P.nodes,
                             pend_grp, Hq);
        stores_done();
        __syncthreads();
        if (tid == 0) {
          int* cnt = P.root_count + (int64_t)pend_s * HT2 + pend_gt;
          const int before = atomicAdd(cnt, 1);
          const int done = before == pend_ngrp - 1;
          if (done) atomicExch(cnt, 0);
          sm_flag[1] = done;
        }
        __syncthreads();
        if (sm_flag[1]) {
          merge_partials<T, D>(P.node_o, P.node_ml, pend_row0, P.nodes, 0, pend_ngrp, pend_nh,
                               (T*)P.out, nullptr, nullptr, 0, 0, Hq);
        }
      }
    }
    pend = false;
  };

  int item = blockIdx.x;
  for (int iter = 0; !planned || item < total; ++iter) {
    // The next item is taken from the queue when wave 0 reaches its last chunk of this
    // one: late enough that items leave the queue in queue order (the long ones first,
    // the short ones last) instead of being held by a workgroup for a whole item while
    // others go idle, and early enough that the answer is back before the epilogue
    // (taking it after the chunk loop instead measured about 1% slower on GQA, MHA and
    // prefix sharing).
#ifdef PA_DECODE_TRACE
    const unsigned long long tr_is = PA_TRACE_STAMP();
    unsigned long long tr_il = 0;
    int tr_tok = 0;  // the item's tokens
#endif
    int next = 0;
    bool took = false;
    auto take_next = [&]() {
      if (tid == 0) next = (int)gridDim.x + atomicAdd(P.queue, 1);
      took = true;
    };

    const bool tiny = planned && item >= A && item < A + Gt;  // uniform over the workgroup
    bool active = true;                             // (tiny) this wave has an item
    int j, gt;
    if (tiny) {
      const int u = NW * (item - A) + wave;
      active = u < c1 * HT2;
      const int uu = active ? u : 0;
      j = jt0 + uu / HT2;
      gt = uu - (uu / HT2) * HT2;
    } else {
      const int idx = !planned || item < A ? item : item - Gt + c1 * HT2;
      j = idx / HT2;
      gt = idx - j * HT2;
    }
    const int g = gt / P.head_tiles;
    const int ht = gt - g * P.head_tiles;
    int s, p;
    if (j < F) {  // a full partition: find s with sm_full[s] <= j < sm_full[s + 1]
      int lo = 0, hi = S;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sm_full[mid] <= j) lo = mid;
        else hi = mid;
      }
      s = lo;
      p = j - sm_full[s];
    } else {  // a sequence's last partition
      s = sm_last[j - F];
      p = -1;
    }
    s = __builtin_amdgcn_readfirstlane(s);
    p = __builtin_amdgcn_readfirstlane(p);
    const int L = __builtin_amdgcn_readfirstlane(sm_len[s]);
    const int hbase = g * P.group + ht * 16;    // first query head of this tile
    const int nh = min(16, P.group - ht * 16);  // query heads in this tile
    const int64_t row0 = (int64_t)s * Hq + hbase;

    if (L <= 0 || L > P.max_tokens) {
      // empty sequence -> zeros; a length the table cannot hold -> NaN rows
      const float fill = L == 0 ? 0.f : __builtin_nanf("");
      T* o = (T*)P.out + row0 * D;
      take_next();
      for (int i = tid; i < nh * D; i += NT_THREADS) o[i] = (T)fill;
    } else {
      const int n = (L + PT - 1) / PT;
      if (p < 0) p = n - 1;
      const int t_begin = p * PT;
      const int t_end = min(L, t_begin + PT);
      // Two workgroups share each compute unit, and the waves of the second one placed
      // there (b >= grid / 2) lose the oldest-first issue arbitration: their first item
      // takes 1.5-2.2x as long as the first workgroup's.  Giving them the higher wave
      // priority for their first item only evens that out where it matters least for
      // the queue order (MHA -2.8%, long context -0.8%, GQA unchanged; same bits).
      if (iter == 0 && blockIdx.x >= gridDim.x / 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      const int nchunks = (t_end - t_begin + 31) >> 5;
#ifdef PA_DECODE_TRACE
      tr_tok = t_end - t_begin;
#endif
      const int last_blk = (L - 1) / BS;  // last table entry the sequence uses

      // query fragment: lane (c, i) holds the same slice of q[head c] that it holds
      // of each key row
      const bool hvalid = col < nh;
      const T* qrow = (const T*)P.q + (row0 + (hvalid ? col : 0)) * D + quad * EPL;
      u32x4 qf[C::KL];
#pragma unroll
      for (int c = 0; c < C::KL; ++c)
        qf[c] = hvalid ? ld16(qrow + c * 4 * EPL) : u32x4{0u, 0u, 0u, 0u};

      const T* kbase = (const T*)P.k_cache + (int64_t)g * tile;
      const T* vbase = (const T*)P.v_cache + (int64_t)g * tile;
      const int32_t AS4* tbl = (const int32_t AS4*)(P.block_tables + (int64_t)s * P.max_blocks);
      // (fused write) this item holds the sequence's last position, whose slot the launch
      // writes: when slot_mapping[s] is that position's slot (checked where the chunk's
      // block ids are at hand), the chunk holding it takes the token's key from k_new (a
      // different load address for the lanes of that row) and its value from vnew, this
      // wave's copy of the v_new row (VW 4-byte words a lane), patched into the value tile
      constexpr int VW = D * (int)sizeof(T) > 256 ? 2 : 1;
      const bool fused_last = FUSE && t_end == L;
      bool red = false;
      int64_t new_slot = -1;
      uint32_t vnew[VW] = {};
      const T* knew_row = nullptr;
      if (fused_last) {
        new_slot = sm_slot[s];
        knew_row = (const T*)P.k_new + ((int64_t)s * P.num_kv_heads + g) * D;
        const uint32_t* vr =
            (const uint32_t*)((const T*)P.v_new + ((int64_t)s * P.num_kv_heads + g) * D);
#pragma unroll
        for (int w = 0; w < VW; ++w)
          vnew[w] = (64 * w + lane) * 4 < D * (int)sizeof(T) ? vr[64 * w + lane] : 0u;
      }

      float m_run = -INFINITY, l_run = 0.f;
      f32x4 acc[NT];
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
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
        if (FUSE && fused_last && t0 + 32 >= L) {  // (uniform) the chunk of the written slot
          int id_last = 0;  // the block id of the last position, one of this chunk's
#pragma unroll
          for (int i = 0; i < IDS; ++i)
            if (j0 + i == last_blk) id_last = ids[i];
          red = new_slot == (int64_t)id_last * BS + (L - 1) % BS;
          if (red && t0 + ka == L - 1) pa = knew_row + quad * EPL;
          if (red && t0 + ka + 4 == L - 1) pb = knew_row + quad * EPL;
        }
#pragma unroll
        for (int k = 0; k < C::KL; ++k) {
          c.ka[k] = ld16_as<NTL>(pa + k * 4 * EPL);
          c.kb[k] = ld16_as<NTL>(pb + k * 4 * EPL);
        }
        if constexpr (BS >= 8) {
          const T* pv = vbase + (int64_t)pick(rv) * blk_stride + vofs;
#pragma unroll
          for (int nn = 0; nn < NT; ++nn)
#pragma unroll
            for (int u = 0; u < C::VL; ++u) c.v[nn][u] = ld16_as<NTL>(pv + nn * 16 * BS + u * EPL);
        } else {  // BS == 4: the 8 tokens straddle two blocks
          const T* lo = vbase + (int64_t)pick(2 * quad) * blk_stride + vofs;
          const T* hi = vbase + (int64_t)pick(2 * quad + 1) * blk_stride + vofs;
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            if constexpr (sizeof(T) == 2) {
              const u32x2 a = ld8(lo + nn * 16 * BS), b = ld8(hi + nn * 16 * BS);
              c.v[nn][0] = u32x4{a[0], a[1], b[0], b[1]};
            } else {
              c.v[nn][0] = ld16_as<NTL>(lo + nn * 16 * BS);
              c.v[nn][1] = ld16_as<NTL>(hi + nn * 16 * BS);
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
        const bool tail = t0 + 32 > t_end;  // uniform: only the last chunk of an item
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
        for (int nn = 0; nn < NT; ++nn) acc[nn] *= alpha;

        if (tail) {  // values past the end may be NaN: zero them, never multiply them
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            if constexpr (sizeof(T) == 2) {
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const uint32_t keep = ((tfirst + 2 * w < t_end) ? 0x0000FFFFu : 0u) |
                                      ((tfirst + 2 * w + 1 < t_end) ? 0xFFFF0000u : 0u);
                c.v[nn][0][w] &= keep;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                c.v[nn][e >> 2][e & 3] = (tfirst + e < t_end) ? c.v[nn][e >> 2][e & 3] : 0u;
            }
          }
        }
        if (FUSE && red && t0 + 32 >= L) {  // (uniform) the written slot's value, from vnew
          const int r = L - 1 - t0;   // its place in the chunk: segment r / 8, element r % 8
          const int e = r & 7;
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            const int d = 16 * nn + col;                  // this lane's dimension
            const int wi = d * (int)sizeof(T) / 4;        // word of the v_new row holding it
            const uint32_t word = (uint32_t)__builtin_amdgcn_ds_bpermute((wi & 63) << 2,
                                                                         (int)vnew[(wi >> 6) % VW]);
            if (quad == (r >> 3)) {
              if constexpr (sizeof(T) == 2) {
                const uint32_t h = (word >> (16 * (d & 1))) & 0xFFFFu;
                const uint32_t x = c.v[nn][0][e >> 1];
                c.v[nn][0][e >> 1] = (e & 1) ? ((x & 0x0000FFFFu) | (h << 16)) : ((x & 0xFFFF0000u) | h);
              } else {  // a static index, so that the chunk buffer stays in registers
#pragma unroll
                for (int x = 0; x < 8; ++x)
                  if (x == e) c.v[nn][x >> 2][x & 3] = word;
              }
            }
          }
        }
        if constexpr (sizeof(T) == 2) {
          // weights as hi + lo pairs of the input type: the sum of two products keeps
          // ~16 significant bits of each fp32 weight, so the weighted sum is as exact
          // as an fp32 one and the only rounding left is the final store
          typedef typename Vec8<T>::type V8;
          V8 phi, plo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const T h = (T)pr[e];
            phi[e] = h;
            plo[e] = (T)(pr[e] - (float)h);
          }
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            const V8 vv = __builtin_bit_cast(V8, c.v[nn][0]);
            acc[nn] = mma16(vv, phi, acc[nn]);
            acc[nn] = mma16(vv, plo, acc[nn]);
          }
        } else {
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            const f32x4 lo = __builtin_bit_cast(f32x4, c.v[nn][0]);
            const f32x4 hi = __builtin_bit_cast(f32x4, c.v[nn][1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[nn] = mma4(lo[e], pr[e], acc[nn]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[nn] = mma4(hi[e], pr[4 + e], acc[nn]);
          }
        }
      };

      // this wave's chunks are wave, wave + NW, ...; two buffers alternate so the
      // next chunk's loads are in flight while this one is computed
      const int nc = tiny ? (active ? 1 : 0) : wave < nchunks ? (nchunks - wave + NW - 1) / NW : 0;
      auto t_of = [&](int i) { return tiny ? 0 : t_begin + 32 * (wave + NW * i); };
      if (nc > 0) {
        C CA, CB;  // the two chunk buffers
        issue(CA, t_of(0));
        // this workgroup's first item: sort while CA loads; a pending arrival is
        // settled here too (the other branch takes the same barriers)
        if (!planned) finish_plan();
        if (pend) settle();
        int i = 0;
        for (; i + 2 < nc; i += 2) {
          issue(CB, t_of(i + 1));
          compute(CA, t_of(i));
          issue(CA, t_of(i + 2));
          compute(CB, t_of(i + 1));
        }
        if (i + 1 < nc) {
          issue(CB, t_of(i + 1));
          compute(CA, t_of(i));
          take_next();
          compute(CB, t_of(i + 1));
        } else {
          take_next();
          compute(CA, t_of(i));
        }
      } else {
        if (!planned) finish_plan();
        if (pend) settle();
      }
      planned = true;
      if (!took) take_next();  // (wave 0 always has a chunk; kept for safety)

#ifdef PA_DECODE_TRACE
      tr_il = PA_TRACE_STAMP();
#endif
      // the epilogue's per-lane indices.  In the fused instance they are recomputed
      // here from an opaque copy of the thread index: hoisted out of the item loop they
      // would be held across the chunk loop, which then spills (measured 1.3% on the
      // fused step; the other instances fit and keep the hoisted form, which measured
      // the same or up to 1.5% faster for them)
      int etid = tid;
      if constexpr (FUSE) asm volatile("" : "+v"(etid));
      const int elane = etid & 63, ecol = elane & 15, equad = elane >> 4;
      if (tiny) {
        // a one-chunk sequence of this wave alone: normalise and store, no merge
        if (active) {
          l_run += __shfl_xor(l_run, 16);
          l_run += __shfl_xor(l_run, 32);
          const bool wbad = __any(bad);
          if (ecol < nh) {
            T* o = (T*)P.out + (row0 + ecol) * D + 4 * equad;
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int nn = 0; nn < NT; ++nn)
              store4(o + 16 * nn, wbad ? f32x4{nan, nan, nan, nan} : acc[nn] / l_run);
          }
        }
      } else {
      // merge the four waves (fixed order) through LDS
      l_run += __shfl_xor(l_run, 16);
      l_run += __shfl_xor(l_run, 32);
      if (equad == 0) {
        sm_m[wave][ecol] = m_run;
        sm_l[wave][ecol] = l_run;
      }
#pragma unroll
      for (int nn = 0; nn < NT; ++nn)
        *reinterpret_cast<f32x4*>(&sm_o[wave][ecol][16 * nn + 4 * equad]) = acc[nn];
      if (elane == 0) sm_bad[wave] = bad;
      __syncthreads();

      int anybad = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) anybad |= sm_bad[w];
      for (int it = etid; it < nh * (D / 4); it += NT_THREADS) {
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
        if (n == 1) {
          store4((T*)P.out + (row0 + hh) * D + d4, O / Ls);
        } else {
          const int64_t slot = ((int64_t)s * P.pmax + p) * Hq + hbase + hh;
          // the item's rows are contiguous: one wave-uniform base, 32-bit offsets
          st_dev16(P.part_o + ((int64_t)s * P.pmax + p) * Hq * D, (int)((hbase + hh) * D + d4) * 4, O);
          if (d4 == 0) st_dev2(P.part_ml + 2 * slot, M, Ls);
        }
      }

      if (n > 1) {
        // publish this partition, then count it in its group of kMergeFan; the answer
        // is read when this workgroup next settles
        stores_done();
        __syncthreads();
        const int grp = p / kMergeFan;
        if (etid == 0)
          pend_before = atomicAdd(P.node_count + ((int64_t)s * HT2 + gt) * P.nodes + grp, 1);
        pend = true;
        pend_s = s;
        pend_gt = gt;
        pend_grp = grp;
        pend_gsize = min(kMergeFan, n - grp * kMergeFan);
        pend_ngrp = (n + kMergeFan - 1) / kMergeFan;
        pend_nh = nh;
        pend_n = n;
        pend_row0 = row0;
      }
      }  // not a one-chunk group
    }

#ifdef PA_DECODE_TRACE
    if (threadIdx.x == 0 && tr_n < kTraceItems) {
      tr[2 + 4 * tr_n] = tr_is;
      tr[3 + 4 * tr_n] = tr_il;
      tr[4 + 4 * tr_n] = PA_TRACE_STAMP();
      tr[5 + 4 * tr_n] = (unsigned long long)(unsigned)item |
                         ((unsigned long long)(tiny ? 1 : 0) << 32) |
                         ((unsigned long long)(planned && item >= A ? 1 : 0) << 33) |
                         ((unsigned long long)tr_tok << 34);
    }
    ++tr_n;
#endif
    // Two slots: thread 0 may write the next item's slot before a slow wave has read
    // this one only if the item in between passes no barrier (the fill path).
    if (!planned) {  // (not reached: the first item of such a workgroup is a full one)
      finish_plan();
      planned = true;
    }
    if (tid == 0) sm_next[iter & 1] = next;
    __syncthreads();  // also: every thread is done with this item's LDS
    item = sm_next[iter & 1];
  }

  if (pend) settle();

#ifdef PA_DECODE_TRACE
  if (threadIdx.x == 0) {
    tr[254] = (unsigned long long)tr_n;
    tr[255] = PA_TRACE_STAMP();
  }
#endif

  // ---------------------------------------------------------------- fused cache write
  // (pa_cache_write_decode) Each sequence's new token goes to its slot, a bit copy of its
  // key row and value column ([RK] 分页注意力是如何工作的: the new token takes the next slot
  // of its sequence's last block).  The stores are done by the workgroups that run out of
  // items first: the k-th to finish stores rows kWriteRows * (k + i * grid), so the last
  // ones to finish have none and the stores fill time the early finishers would sit idle.
  // Nothing in this launch reads a slot written here: the chunk that holds a sequence's
  // last position took that token's key and value from k_new / v_new (see `red`).
  int finished_before = 0;  // (thread 0, and every thread when FUSE) workgroups finished before this one
  if (tid == 0) finished_before = atomicAdd(P.queue + 1, 1);
  if constexpr (FUSE) {
    if (tid == 0) sm_flag[0] = finished_before;
    __syncthreads();
    finished_before = sm_flag[0];
    constexpr int KP = D * (int)sizeof(T) / 16;  // 16-byte pieces of a key row
    const int Hkv = P.num_kv_heads;
    const int rows = S * Hkv;                    // (token, KV head) rows
    for (int r0 = finished_before * kWriteRows; r0 < rows; r0 += (int)gridDim.x * kWriteRows) {
      const int nr = min(kWriteRows, rows - r0);
      for (int u = tid; u < nr * KP; u += NT_THREADS) {
        const int64_t iu = r0 + u / KP;
        const int piece = u % KP;
        const int64_t slot = P.slot_mapping[iu / Hkv];
        if (slot < 0 || slot >= P.num_slots) continue;
        const int64_t g = iu % Hkv;
        T* dst = (T*)P.k_cache + (((slot / BS) * Hkv + g) * BS + slot % BS) * D + piece * EPL;
        *reinterpret_cast<u32x4*>(dst) = ld16((const T*)P.k_new + iu * D + piece * EPL);
      }
      for (int u = tid; u < nr * D; u += NT_THREADS) {
        const int64_t iu = r0 + u / D;
        const int d = u % D;
        const int64_t slot = P.slot_mapping[iu / Hkv];
        if (slot < 0 || slot >= P.num_slots) continue;
        const int64_t g = iu % Hkv;
        ((T*)P.v_cache)[(((slot / BS) * Hkv + g) * D + d) * BS + slot % BS] =
            ((const T*)P.v_new)[iu * D + d];
      }
    }
  }

  // the last workgroup out resets the queue for the next call
  if (tid == 0 && finished_before == (int)gridDim.x - 1) {
    atomicExch(P.queue, 0);
    atomicExch(P.queue + 1, 0);
  }
}

// FUSE: the instance behind pa_cache_write_decode (new tokens stored in the same launch)
template <typename T, int D, int BS>
const void* kernel_of(bool stream_kv, bool fuse) {
  if (fuse)
    return stream_kv ? (const void*)decode_kernel<T, D, BS, true, true>
                     : (const void*)decode_kernel<T, D, BS, false, true>;
  return stream_kv ? (const void*)decode_kernel<T, D, BS, true, false>
                   : (const void*)decode_kernel<T, D, BS, false, false>;
}

template <typename T, int D>
const void* kernel_bs(int bs, bool nt, bool fu) {
  switch (bs) {
    case 4: return kernel_of<T, D, 4>(nt, fu);
    case 8: return kernel_of<T, D, 8>(nt, fu);
    case 16: return kernel_of<T, D, 16>(nt, fu);
    case 32: return kernel_of<T, D, 32>(nt, fu);
  }
  return nullptr;
}

template <typename T>
const void* kernel_d(int d, int bs, bool nt, bool fu) {
  switch (d) {
    case 64: return kernel_bs<T, 64>(bs, nt, fu);
    case 128: return kernel_bs<T, 128>(bs, nt, fu);
  }
  return nullptr;
}

const void* decode_kernel_for(int dtype, int head_dim, int block_size, bool nt, bool fu) {
  switch (dtype) {
    case 0: return kernel_d<float>(head_dim, block_size, nt, fu);
    case 1: return kernel_d<_Float16>(head_dim, block_size, nt, fu);
    case 2: return kernel_d<__bf16>(head_dim, block_size, nt, fu);
  }
  return nullptr;
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int block_size, const DecodeParams& p,
                         int grid, hipStream_t stream) {
  const void* k = decode_kernel_for(dtype, head_dim, block_size, p.stream_kv != 0,
                                    p.slot_mapping != nullptr);
  if (!k || grid <= 0) return hipErrorInvalidValue;
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(k, dim3(grid), dim3(NT_THREADS), args, 0, stream);
}

hipError_t decode_blocks_per_cu(int dtype, int head_dim, int block_size, int* blocks) {
  // the cache-policy and fused-write variants are all compiled for the same workgroups
  // per compute unit (their launch bounds)
  const void* k = decode_kernel_for(dtype, head_dim, block_size, true, false);
  if (!k) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, NT_THREADS, 0);
}

}  // namespace pa

#ifdef PA_DECODE_TRACE
// (diagnostic build) copy the trace buffer of the last decode launch to host memory
extern "C" __attribute__((visibility("default"))) int pa_decode_trace_read(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(pa::pa_trace_buf),
                                  bytes < sizeof(pa::pa_trace_buf) ? bytes : sizeof(pa::pa_trace_buf),
                                  0, hipMemcpyDeviceToHost);
}
#endif
