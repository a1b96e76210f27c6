// Ragged paged attention for gfx950 (CDNA4): planning prepass, decode / split-KV kernel,
// prefill-chunk kernel and the log-sum-exp merge.
//
// What is computed (the pages give no formula; scaled dot-product softmax attention is the
// reading): the token at position p of sequence s attends to keys 0..p of s only — ragged
// batching with a block-diagonal mask ("Continuous batching from first principles",
// Takeaways) and chunked prefill attending to a cache that already holds earlier chunks
// ("3.3 Batching & Memory Management", section "Chunked prefill"). Keys and values are
// gathered through the block table ("PagedAttention: block tables").
//
// Work split. A sequence whose rows (new tokens x query heads per KV head, G = Hq/Hkv) fit in
// one 16-row MFMA tile (q * G <= 16) is decode-type: its KV range is cut into partitions of P
// tokens, and each (partition, KV head) item is streamed by one wave of a persistent decode
// grid that takes items from a queue; several partitions are merged afterwards by log-sum-exp.
// A small decode-only batch has no planning launch: the decode waves derive their items (and
// write the step's K/V rows) themselves.
// Longer chunks are prefill-type: one 8-wave workgroup per (256-row query tile, KV head) over
// the tile's causal key range (split along the keys into parts when the batch has too few
// tiles to fill the GPU), with 32-key K/V tiles staged in LDS and read by all 8 waves.
//
// MFMA orientation (both kernels): the key dimension is the A operand's row index,
//   S^T[key][row]  = K[key][:] . Q[row][:]        (A = K rows, B = Q^T, contraction over dims)
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row] (A = V^T,   B = P^T, contraction over keys)
// so each output lane holds one query row (its column of S^T and O^T): the running max and sum
// are lane-local up to one cross-lane step, the rescale of O needs no data movement, and the
// probabilities leave the first MFMA already in the B layout of the second. The contraction
// index may be permuted freely as long as A and B agree. Decode: v_mfma_f32_16x16x32_bf16 on
// 16 keys x (up to 16 query rows); its V^T operand is built in registers from 16-byte pieces
// of 8 dims of one key with byte permutes. Prefill: v_mfma_f32_32x32x16_bf16 on 32 keys x 32
// query rows per wave; its V^T operand comes from transposing LDS reads.
//
// Masking is by select before the exponential (never by multiplying with 0), and V rows of
// keys at or past the range end are zeroed, so NaN or stale data in unread slots (block tails,
// unassigned blocks) cannot reach the output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "cb_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima start at this finite floor so that exp2(m_old - m_new) never sees inf - inf.
constexpr float kMaxFloor = -1e30f;
constexpr int kMaxSplitTokens = 2048;  // partition size cap: <= 129 table entries at bs 16
constexpr int kPrefillWaves = 8;                   // waves per prefill workgroup, 2 per SIMD
constexpr int kPrefillRows = kPrefillWaves * 32;   // query rows (token x head) per tile: 32 per wave
constexpr int kPrefillWavesPerSimd = 2;
constexpr int kDecodeWaves = 8;  // waves per decode workgroup beside prefill work (4 otherwise)

// A prefill item carries what its workgroup needs to start (one 32-byte scalar load): sequence,
// query tile * kMaxPreSplits + key part, the sequence's first packed row, query rows, KV length.
struct alignas(16) Work {
  int32_t seq, idx, q0, qn, L, pad0, pad1, pad2;
};
// A decode item carries what its wave needs to start (one 32-byte scalar load): sequence, KV
// partition, first query row, query rows, KV length.
struct alignas(32) DecWork {
  int32_t seq, split, q0, qn, L, pad0, pad1, pad2;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS transpose read of 4 x 16-bit per lane: within each 16-lane group, lane 4a + b receives
// element b of the 8-byte reads of lanes a, 4 + a, 8 + a and 12 + a (in that order).
__device__ inline s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

template <bool B>
struct Tag {
  static constexpr bool value = B;
};
template <int X>
struct Int {
  static constexpr int value = X;
};

__device__ inline f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Reductions over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with the row-swap
// permutes: permlane16_swap(x, x) yields the values of the even and the odd 16-lane row of each
// row pair, permlane32_swap(x, x) those of the lower and the upper 32 lanes.
__device__ inline float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The running reference max of a row moves only when a chunk's max exceeds it by more than this
// (log2 units): probabilities are then bounded by 2^8, and the rescale of O is skipped for most
// chunks. The result is unchanged: numerator and denominator share the reference.
constexpr float kRescaleSlack = 8.f;

// Fragments of one 32-key step for one lane.
template <int D>
struct KVFrag {
  static constexpr int KSTEPS = D / 32;  // MFMA k-steps over the head dimension
  static constexpr int DW = D / 32;      // 32-bit words of V per key per lane (D/16 bf16)
  bf16x8 k[2][KSTEPS];                   // K: key group j (16 keys), k-step kk
  uint32_t v[8][DW];                     // V: key e = 16*(e/4) + 4g + e%4, dims n*D/16 ..
};

// Online softmax of one 16-row tile over one 32-key chunk, in three parts.
//   acc[j][i]: raw score (Q.K) for key k0 + 16j + 4g + i of this lane's row; c = scale * log2(e).
// m is the row's reference max in scaled log2 units (the same in the row's four lanes), l this
// lane's part of the row's running sum (the row sum is the sum over the four lanes, taken once
// at the end: every rescale multiplies all four parts by the same factor), o its output rows.

// This lane's max over its 8 keys of the chunk (scaled). With MASK, keys >= kend or > last_key are
// first set to -inf in acc; without it the caller guarantees every key of the chunk is visible to
// every row that is written out.
template <bool MASK>
__device__ inline float chunk_max(f32x4 (&acc)[2], int k0, int kend, int last_key, float c, int g) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (MASK) {
        const int key = k0 + 16 * j + 4 * g + i;
        acc[j][i] = (key < kend && key <= last_key) ? acc[j][i] : -INFINITY;
      }
      mx = fmaxf(mx, acc[j][i]);
    }
  }
  return mx * c;  // c > 0; -inf stays -inf
}

// Move the reference max when some lane's chunk max exceeds it by more than kRescaleSlack; only
// then is the row max over the four lanes taken.
template <int NO>
__device__ inline void rescale_lazy(float m_lane, float& m, float& l, f32x4 (&o)[NO]) {
  if (__builtin_amdgcn_ballot_w64(m_lane > m + kRescaleSlack) != 0) {  // wave-uniform
    const float m_new = fmaxf(m, group_max(m_lane));
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < NO; ++t) o[t] *= alpha;
    m = m_new;
  }
}

// Probabilities of the chunk against the reference max, added to this lane's part of the sum;
// returns P^T (bf16) in the B-operand layout. Masked scores are -inf and give 0.
__device__ inline bf16x8 chunk_exp(const f32x4 (&acc)[2], float c, float m, float& l) {
  float rs = 0.f;
  bf16x8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e >> 2][e & 3], c, -m));
    rs += p;
    pb[e] = (__bf16)p;
  }
  l += rs;
  return pb;
}

template <int NO, bool MASK>
__device__ inline bf16x8 softmax_step(f32x4 (&acc)[2], int k0, int kend, int last_key,
                                      float c, int g, float& m, float& l, f32x4 (&o)[NO]) {
  const float m_chunk = chunk_max<MASK>(acc, k0, kend, last_key, c, g);
  rescale_lazy<NO>(m_chunk, m, l, o);
  return chunk_exp(acc, c, m, l);
}

// V^T operand of output tile jt: element e = V[key e][dim n*D/16 + jt], from 8 keys' words.
// perm(hi, lo, 0x05040100) = lo16(lo) | lo16(hi) << 16; perm(hi, lo, 0x07060302) = the high halves.
template <int D>
__device__ inline bf16x8 vt_operand(const uint32_t (&v)[8][D / 32], int jt) {
  const int w = jt >> 1;
  const uint32_t sel = (jt & 1) ? 0x07060302u : 0x05040100u;
  uint32_t d[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) d[a] = __builtin_amdgcn_perm(v[2 * a + 1][w], v[2 * a][w], sel);
  return __builtin_bit_cast(bf16x8, d);
}

// ---------------------------------------------------------------------------------------------
// Planning prepass: per-sequence work items, compacted with a block-wide scan.

// A sequence breaking the contract (q = 0, kv_len < q, kv_len beyond max_kv_len, more KV than its
// table row addresses, a decode-type q beyond max_q_len) gets no work item, so nothing is read
// or written out of bounds; its output rows are then left unwritten.
//
// Decode items are ordered longest first, so that the work queue ends on short items: every
// full P-token partition first (in sequence order), then each sequence's last, partial
// partition, bucketed by decreasing length. Prefill items: a sequence's last query tiles (they
// see the most keys) first.
constexpr int kTailBuckets = 32;

// Prefill tiles are split along the keys when the batch has too few prefill workgroups to fill
// the GPU (fewer than two per compute unit): a tile of kend keys becomes ns parts of `chunk`
// keys (a multiple of 32), one part per kPrefillSplitKeys keys, at most emax parts. Parts write
// fp32 (o, lse) partials that the log-sum-exp merge combines. Plan and kernel use this same
// function, so they agree on the parts.
constexpr int kMaxPreSplits = 4;
constexpr int kPrefillSplitKeys = 1536;
// Splitting pays only when the longest prefill tile would outlast the batch's decode work, which
// otherwise fills the compute units that the long tiles leave idle (the two kernels run side by
// side). Estimated from measured rates on this GPU: one 32-key step of a prefill workgroup takes
// about 1.0 us, and the decode kernel streams about 5.5 GB/ms.
constexpr float kPrefillStepUs = 1.0f;
constexpr float kDecodeBytesPerUs = 5.5e6f;

__device__ inline void prefill_split(int kend, int emax, int& ns, int& chunk) {
  int n0 = emax > 1 ? min(emax, (kend + kPrefillSplitKeys - 1) / kPrefillSplitKeys) : 1;
  if (n0 < 1) n0 = 1;
  chunk = ((kend + n0 - 1) / n0 + 31) / 32 * 32;
  ns = (kend + chunk - 1) / chunk;
}

// A sequence's inputs to the plan: first packed row, query rows and KV length (zeros past the
// last sequence, which then has no work).
struct SeqIn {
  int c0, q, L;
};
__device__ __forceinline__ SeqIn seq_in(const int32_t* __restrict__ cu,
                                        const int32_t* __restrict__ kv_lens, int s, int num_seqs) {
  if (s >= num_seqs) return SeqIn{0, 0, 0};
  const int c0 = cu[s];
  return SeqIn{c0, cu[s + 1] - c0, kv_lens[s]};
}

__device__ inline int seq_items(const SeqIn& in, int G, int P, int qmaxd, int max_splits, int bq,
                                int bs, int max_blocks, int max_kv, int& nfull, int& rem, int& np) {
  nfull = 0;
  rem = 0;
  np = 0;
  const int q = in.q, L = in.L;
  if (q <= 0 || L < q || L > max_kv || (L + bs - 1) / bs > max_blocks) return 0;
  if (q * G <= 16) {
    if (q > qmaxd || (L + P - 1) / P > max_splits) return 0;
    nfull = L / P;
    rem = L - nfull * P;
  } else {
    np = (q + bq - 1) / bq;
  }
  return 1;
}

// Sum over the wave's lanes (64-bit, as two 32-bit halves per shuffle).
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    v += (unsigned long long)hi << 32 | lo;
  }
  return v;
}

// Inclusive prefix sums of two values over the 1024 threads of the planning workgroup: within
// each wave by shuffles, then over the 16 wave totals by the first wave. Two barriers; wsum
// ([16], shared) may be reused after the caller's next barrier.
__device__ __forceinline__ int2 block_scan2(int a, int b, int2* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ya = __shfl_up(a, off, 64), yb = __shfl_up(b, off, 64);
    if (lane >= off) {
      a += ya;
      b += yb;
    }
  }
  if (lane == 63) wsum[w] = make_int2(a, b);
  __syncthreads();
  if (w == 0) {
    int2 v = lane < 16 ? wsum[lane] : make_int2(0, 0);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int ya = __shfl_up(v.x, off, 64), yb = __shfl_up(v.y, off, 64);
      if (lane >= off) {
        v.x += ya;
        v.y += yb;
      }
    }
    if (lane < 16) wsum[lane] = v;
  }
  __syncthreads();
  if (w > 0) {
    a += wsum[w - 1].x;
    b += wsum[w - 1].y;
  }
  return make_int2(a, b);
}

__device__ __forceinline__ void plan_body(const int32_t* __restrict__ cu,
                                          const int32_t* __restrict__ kv_lens,
                                          int32_t num_seqs, int32_t G, int32_t P,
                                          int32_t qmaxd, int32_t max_splits,
                                          int32_t bq, int32_t bs, int32_t max_blocks,
                                          int32_t max_kv, DecWork* __restrict__ dec,
                                          int64_t dec_cap, Work* __restrict__ pre,
                                          int64_t pre_cap, int32_t* __restrict__ counts,
                                          int32_t Hkv, int32_t cus, int32_t maxs,
                                          int32_t num_tokens, int32_t kv_token_bytes,
                                          int32_t* __restrict__ nsplit_tok, int32_t beside) {
  __shared__ int2 wsum[16];
  __shared__ int32_t first_item[1024];  // index of each thread's first full partition
  __shared__ int32_t sh_c0[1024], sh_q[1024], sh_L[1024];  // this pass's sequences' inputs
  __shared__ int32_t base[2];
  __shared__ int32_t split_on;
  __shared__ int32_t pre_tiles;            // prefill tiles of the batch
  __shared__ unsigned long long dec_keys;  // sum of decode sequences' lengths
  __shared__ unsigned long long pre_steps; // 32-key steps of all prefill tiles (one KV head)
  __shared__ int32_t max_pre_len;          // longest prefill sequence (its last tile's keys)
  __shared__ int32_t tail_count[kTailBuckets];
  __shared__ int32_t tail_next[kTailBuckets];
  const int tid = threadIdx.x;
  // Up to 1024 sequences (one per thread) are planned in one pass, and each thread keeps its
  // sequence's inputs and item counts in registers for the later passes; more take one pass per
  // 1024 sequences, each reading its inputs again.
  const bool one = num_seqs <= 1024;
  if (tid == 0) {
    base[0] = base[1] = 0;
    dec_keys = 0;
    pre_steps = 0;
    max_pre_len = 0;
  }
  if (tid < kTailBuckets) tail_count[tid] = tail_next[tid] = 0;
  if (maxs > 1)  // split counts of prefill tokens: 0 until a split tile writes its own
    for (int t = tid; t < num_tokens; t += 1024) nsplit_tok[t] = 0;
  __syncthreads();
  SeqIn in{0, 0, 0};
  int nfull = 0, rem = 0, np = 0;
  // pass 1: full partitions by prefix sums; prefill tiles counted; tails counted per bucket
  for (int s0 = 0; s0 < num_seqs; s0 += 1024) {
    const int s = s0 + tid;
    in = seq_in(cu, kv_lens, s, num_seqs);
    seq_items(in, G, P, qmaxd, max_splits, bq, bs, max_blocks, max_kv, nfull, rem, np);
    sh_c0[tid] = in.c0;
    sh_q[tid] = in.q;
    sh_L[tid] = in.L;
    if (rem > 0) atomicAdd(&tail_count[(P - rem) * kTailBuckets / P], 1);
    // decode keys: a wave's sum, then one shared atomic per wave
    const unsigned long long dk = wave_sum_u64((unsigned long long)(nfull * P + rem));
    if ((tid & 63) == 0 && dk > 0) atomicAdd(&dec_keys, dk);
    if (np > 0) {
      atomicMax(&max_pre_len, in.L);
      // 32-key steps of the sequence's query tiles: tile t sees keys [0, L - q + min(q, (t + 1) bq)).
      // With bq a multiple of 32 the full tiles 0 .. np - 2 add bq / 32 steps each to the first
      // one's ceil((L - q) / 32) + bq / 32 (closed form instead of a loop over the tiles, which
      // took microseconds for long chunks); the last tile sees all L keys.
      unsigned long long stp = 0;
      if ((bq & 31) == 0) {
        const unsigned long long m = (unsigned long long)(np - 1);
        stp = m * (unsigned long long)((in.L - in.q + 31) / 32) +
              (unsigned long long)(bq / 32) * m * (m + 1) / 2 + (unsigned long long)((in.L + 31) / 32);
      } else {
        for (int t = 0; t < np; ++t) stp += (in.L - in.q + min(in.q, (t + 1) * bq) + 31) / 32;
      }
      atomicAdd(&pre_steps, stp);
    }
    const int2 inc = block_scan2(nfull, np, wsum);
    first_item[tid] = inc.x - nfull;
    __syncthreads();
    // The full partitions of these 1024 sequences, written by all threads: item i belongs to the
    // last thread t with first_item[t] <= i (threads with no full partition share the next one's
    // first index, so the last such t has one), as partition i - first_item[t] of sequence s0 + t.
    const int total_items = wsum[15].x;
    for (int i = tid; i < total_items; i += 1024) {
      int lo = 0, hi = 1023;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first_item[mid] <= i) lo = mid; else hi = mid - 1;
      }
      const int64_t ed = (int64_t)base[0] + i;
      if (ed < dec_cap)
        dec[ed] = DecWork{s0 + lo, i - first_item[lo], sh_c0[lo], sh_q[lo], sh_L[lo], 0, 0, 0};
    }
    __syncthreads();
    if (tid == 1023) {
      base[0] += inc.x;
      base[1] += inc.y;
    }
    __syncthreads();
  }
  // bucket offsets after the full partitions (bucket 0 holds the longest tails)
  if (tid == 0) {
    int acc = base[0];
    for (int b = 0; b < kTailBuckets; ++b) {
      tail_next[b] = acc;
      acc += tail_count[b];
    }
    counts[0] = (int32_t)min((int64_t)acc, dec_cap);
    counts[2] = 0;  // decode work-queue head
    pre_tiles = base[1];
    base[1] = 0;  // prefill item offset
    if (pre_tiles == 0) counts[1] = 0;
    const float t_decode = (float)dec_keys * Hkv * kv_token_bytes / kDecodeBytesPerUs;
    const float t_longest = (float)((max_pre_len + 31) / 32) * kPrefillStepUs;
    split_on = (maxs > 1 && (int64_t)pre_tiles * Hkv < 2 * (int64_t)cus && t_longest > t_decode)
                   ? 1 : 0;  // split prefill tiles
    counts[3] = split_on;
    // Compute units for the decode kernel when it runs beside the prefill kernel (one workgroup
    // each): its share of the estimated work, at least half of them (below that its streaming
    // rate drops). Without prefill work, or when the decode kernel runs after the prefill kernel
    // on the same stream (beside = 0), every workgroup of the decode grid works.
    const float t_prefill = (float)pre_steps * Hkv * kPrefillStepUs / cus;
    int n_dec = 1 << 30;
    if (beside && t_prefill > 0.f && t_decode > 0.f)
      n_dec = max(cus / 2, min(cus, (int)(cus * t_decode / (t_decode + t_prefill) + 0.5f)));
    counts[4] = n_dec;
  }
  __syncthreads();
  const int emax = split_on ? maxs : 1;
  // prefill items (sequence, tile * kMaxPreSplits + part): a sequence's last tiles first
  if (pre_tiles > 0) {
    for (int s0 = 0; s0 < num_seqs; s0 += 1024) {
      const int s = s0 + tid;
      SeqIn pin = in;
      int pf, pr, pn = np;
      if (!one) {
        pin = seq_in(cu, kv_lens, s, num_seqs);
        seq_items(pin, G, P, qmaxd, max_splits, bq, bs, max_blocks, max_kv, pf, pr, pn);
      }
      const int qn = pin.q, L = pin.L;
      int nit = pn;
      if (pn > 0 && emax > 1) {  // few tiles (splitting is on): count the parts
        nit = 0;
        for (int tl = 0; tl < pn; ++tl) {
          int ns, chunk;
          prefill_split(L - qn + min(qn, (tl + 1) * bq), emax, ns, chunk);
          nit += ns;
        }
      }
      const int incp = block_scan2(nit, 0, wsum).x;
      int64_t ep = (int64_t)base[1] + incp - nit;
      if (emax > 1) {  // few tiles: each sequence's thread writes its tiles' parts
        for (int tl = pn - 1; tl >= 0; --tl) {
          int ns, chunk;
          prefill_split(L - qn + min(qn, (tl + 1) * bq), emax, ns, chunk);
          for (int part = 0; part < ns; ++part, ++ep)
            if (ep < pre_cap) pre[ep] = Work{s, tl * kMaxPreSplits + part, pin.c0, qn, L, 0, 0, 0};
        }
      } else {
        // one item per tile, written by all threads as the full decode partitions are: item i
        // belongs to the last thread t with first_item[t] <= i, as tile pn_t - 1 - (i -
        // first_item[t]) of its sequence (a long chunk's tiles, one thread each, took
        // microseconds)
        first_item[tid] = incp - nit;
        sh_c0[tid] = pin.c0;
        sh_q[tid] = qn;
        sh_L[tid] = L;
        __syncthreads();
        const int pass_items = wsum[15].x;
        for (int i = tid; i < pass_items; i += 1024) {
          int lo = 0, hi = 1023;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first_item[mid] <= i) lo = mid; else hi = mid - 1;
          }
          const int pn_lo = (sh_q[lo] + bq - 1) / bq;
          const int64_t ed = (int64_t)base[1] + i;
          if (ed < pre_cap)
            pre[ed] = Work{s0 + lo, (pn_lo - 1 - (i - first_item[lo])) * kMaxPreSplits, sh_c0[lo],
                           sh_q[lo], sh_L[lo], 0, 0, 0};
        }
      }
      __syncthreads();
      if (tid == 1023) base[1] += incp;
      __syncthreads();
    }
    if (tid == 0) counts[1] = (int32_t)min((int64_t)base[1], pre_cap);
  }
  // pass 2: place the tails (tail_next is set and visible since the barrier above)
  for (int s0 = 0; s0 < num_seqs; s0 += 1024) {
    const int s = s0 + tid;
    if (!one) {
      in = seq_in(cu, kv_lens, s, num_seqs);
      seq_items(in, G, P, qmaxd, max_splits, bq, bs, max_blocks, max_kv, nfull, rem, np);
    }
    if (rem > 0) {
      const int64_t pos = atomicAdd(&tail_next[(P - rem) * kTailBuckets / P], 1);
      if (pos < dec_cap) dec[pos] = DecWork{s, nfull, in.c0, in.q, in.L, 0, 0, 0};
    }
  }
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ cu,
                                                    const int32_t* __restrict__ kv_lens,
                                                    int32_t num_seqs, int32_t G, int32_t P,
                                                    int32_t qmaxd, int32_t max_splits,
                                                    int32_t bq, int32_t bs, int32_t max_blocks,
                                                    int32_t max_kv, DecWork* __restrict__ dec,
                                                    int64_t dec_cap, Work* __restrict__ pre,
                                                    int64_t pre_cap, int32_t* __restrict__ counts,
                                                    int32_t Hkv, int32_t cus, int32_t maxs,
                                                    int32_t num_tokens, int32_t kv_token_bytes,
                                                    int32_t* __restrict__ nsplit_tok,
                                                    int32_t beside) {
  plan_body(cu, kv_lens, num_seqs, G, P, qmaxd, max_splits, bq, bs, max_blocks, max_kv, dec,
            dec_cap, pre, pre_cap, counts, Hkv, cus, maxs, num_tokens, kv_token_bytes, nsplit_tok,
            beside);
}

// The step's cache write with its slots computed in place: the new K/V row of packed token t of
// sequence s (cu[s] <= t < cu[s + 1]) goes to position p = kv_lens[s] - q_s + (t - cu[s]), slot
// table[s][p / bs] * bs + p % bs ("3.3 Batching & Memory Management", PagedAttention: block
// tables). Rows with no valid position or slot (p < 0, past the table row, a negative or
// out-of-pool block) are skipped, as the slot mapping's -1 is. One wave per token (grid-stride):
// the wave finds the token's sequence, then its lanes copy the K and V rows 16 bytes each.
struct WriteArgs {
  const uint4* k;
  const uint4* v;
  uint4* k_cache;
  uint4* v_cache;
  const int32_t* tables;
  int32_t chunks;     // 16-byte chunks per token row (Hkv * D * 2 / 16)
  int64_t slots;      // num_blocks * bs
};

// The sequence of packed token t (0 <= t < cu[num_seqs], num_seqs >= 1): the last s < num_seqs
// with cu[s] <= t. cu is non-decreasing and cu[0] = 0, so the entries <= t form a prefix and s is
// their count minus one. Up to 1024 sequences: each lane loads up to 16 entries at once and the
// wave counts them (one round of loads). More: the lanes compare 64 evenly spaced entries and the
// range shrinks 64-fold per round. Only cu[0 .. num_seqs) is read.
__device__ __forceinline__ int seq_of_token(const int32_t* __restrict__ cu, int num_seqs, int t,
                                            int lane) {
  if (num_seqs <= 1024) {
    const int per = (num_seqs + 63) >> 6;  // entries per lane, 1..16
    int v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = lane * per + j;
      v[j] = (j < per && i < num_seqs) ? cu[i] : INT32_MAX;
    }
    int n = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[j] <= t));
    return n - 1;
  }
  int lo = 0, len = num_seqs;  // cu[lo] <= t holds throughout (cu[0] = 0)
  while (len > 1) {
    const int step = (len + 63) / 64;
    const bool ok = lane * step < len && cu[lo + lane * step] <= t;
    const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok)) - 1;
    lo += k * step;
    len = min(step, len - k * step);
  }
  return lo;
}

// The token's K and V rows are loaded first (they depend on t alone), so their latency overlaps
// the sequence search and the table lookup that give the slot.
__device__ __forceinline__ void write_body(const WriteArgs& w, const int32_t* __restrict__ cu,
                                           const int32_t* __restrict__ kv_lens, int32_t num_seqs,
                                           int32_t num_tokens, int32_t bs, int32_t max_blocks,
                                           int first_wave, int num_waves) {
  const int lane = threadIdx.x & 63;
  for (int t = first_wave; t < num_tokens; t += num_waves) {
    if (w.chunks <= 256) {  // a row of at most 4 KiB: four 16-byte pieces per lane
      const u32x4* kin = reinterpret_cast<const u32x4*>(w.k) + (int64_t)t * w.chunks;
      const u32x4* vin = reinterpret_cast<const u32x4*>(w.v) + (int64_t)t * w.chunks;
      u32x4 kr[4], vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // pieces past the row end load its last piece (not stored)
        const int c = min(lane + 64 * r, w.chunks - 1);
        kr[r] = kin[c];
        vr[r] = vin[c];
      }
      const int s = seq_of_token(cu, num_seqs, t, lane);
      const int32_t q = cu[s + 1] - cu[s];
      const int32_t p = kv_lens[s] - q + (t - cu[s]);
      if (p < 0) continue;
      const int32_t j = p / bs;
      if (j >= max_blocks) continue;
      const int32_t blk = w.tables[(int64_t)s * max_blocks + j];
      const int64_t slot = (int64_t)blk * bs + p % bs;
      if (blk < 0 || slot >= w.slots) continue;
      u32x4* kout = reinterpret_cast<u32x4*>(w.k_cache) + slot * w.chunks;
      u32x4* vout = reinterpret_cast<u32x4*>(w.v_cache) + slot * w.chunks;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = lane + 64 * r;
        if (c < w.chunks) {
          kout[c] = kr[r];
          vout[c] = vr[r];
        }
      }
      continue;
    }
    const int s = seq_of_token(cu, num_seqs, t, lane);
    const int32_t q = cu[s + 1] - cu[s];
    const int32_t p = kv_lens[s] - q + (t - cu[s]);
    if (p < 0) continue;
    const int32_t j = p / bs;
    if (j >= max_blocks) continue;
    const int32_t blk = w.tables[(int64_t)s * max_blocks + j];
    const int64_t slot = (int64_t)blk * bs + p % bs;
    if (blk < 0 || slot >= w.slots) continue;
    for (int c = lane; c < w.chunks; c += 64) {
      w.k_cache[slot * w.chunks + c] = w.k[(int64_t)t * w.chunks + c];
      w.v_cache[slot * w.chunks + c] = w.v[(int64_t)t * w.chunks + c];
    }
  }
}

// Workgroup 0 plans the attention work while the other workgroups write the step's K/V into the
// cache: the plan does not read the cache, so the two need not wait for each other.
__global__ __launch_bounds__(1024) void plan_write_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ kv_lens, int32_t num_seqs,
    int32_t G, int32_t P, int32_t qmaxd, int32_t max_splits, int32_t bq, int32_t bs,
    int32_t max_blocks, int32_t max_kv, DecWork* __restrict__ dec, int64_t dec_cap,
    Work* __restrict__ pre, int64_t pre_cap, int32_t* __restrict__ counts, int32_t Hkv,
    int32_t cus, int32_t maxs, int32_t num_tokens, int32_t kv_token_bytes,
    int32_t* __restrict__ nsplit_tok, int32_t beside, WriteArgs w) {
  if (blockIdx.x == 0) {
    plan_body(cu, kv_lens, num_seqs, G, P, qmaxd, max_splits, bq, bs, max_blocks, max_kv, dec,
              dec_cap, pre, pre_cap, counts, Hkv, cus, maxs, num_tokens, kv_token_bytes, nsplit_tok,
              beside);
    return;
  }
  const int wpb = (int)(blockDim.x >> 6);
  write_body(w, cu, kv_lens, num_seqs, num_tokens, bs, max_blocks,
             __builtin_amdgcn_readfirstlane((int)(blockIdx.x - 1) * wpb + (int)(threadIdx.x >> 6)),
             (int)(gridDim.x - 1) * wpb);
}

// Division of keys (0 <= key < 2^31) by the block size with a multiply and a shift. With
// l = ceil(log2 bs) and magic = ceil(2^(31 + l) / bs), which is below 2^32, key / bs equals
// floor(key * magic / 2^(31 + l)) exactly (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994: the error of the scaled reciprocal stays below 1 / bs).
// The kernel takes the high 32 bits of the product and shifts them right by l - 1.
struct BlockDiv {
  int32_t bs;
  uint32_t magic;
  int32_t shift;
  __device__ int div(int key) const { return (int)(__umulhi((uint32_t)key, magic) >> shift); }
};
inline BlockDiv block_div(int32_t bs) {
  int l = 0;
  while ((1 << l) < bs) ++l;
  const uint64_t num = uint64_t{1} << (31 + l);
  return BlockDiv{bs, (uint32_t)((num + (uint64_t)bs - 1) / (uint64_t)bs), l - 1};
}

// ---------------------------------------------------------------------------------------------
// Decode / split-KV kernel. Persistent waves, each working alone: a wave takes one
// (KV partition, KV head) item at a time from a queue and streams its keys 32 at a time. K/V
// fragments go straight from HBM into registers with 16-byte loads, two steps ahead of the
// MFMAs (each register set is refilled as soon as its MFMAs have read it); the partition's block
// ids sit one per lane and are broadcast with readlane. No LDS and no barriers, so a wave's
// start-up and write-out overlap with the other waves' streaming.

// K/V rows of one 16-key group are read through a buffer resource whose record count ends at the
// range end: loads of keys at or past it return zeros and touch no memory, so a step's loads need
// no branch and V rows past the end arrive zeroed (their slots may hold anything, NaN included).
// The address and count are wave-uniform; readfirstlane puts them in scalar registers, where
// the descriptor must be (from vector registers the compiler would loop over the lanes).
__device__ inline __amdgpu_buffer_rsrc_t group_rsrc(const __bf16* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>((uint64_t)hi << 32 | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(nbytes),
                                           0x00020000);
}
constexpr int kLoadStream = 2;  // buffer-load cache policy: non-temporal (K/V are read once)

// The loads of one 32-key step into registers. K: lane (n, g) reads dims [32 kk + 8 g, +8) of key
// 16 j + n, so one instruction covers 64 contiguous bytes of each of 16 key rows and the next one
// completes each 128-byte line: ordinary cached loads. V: lane (c = n, g) reads chunk n of key
// 16 (e / 4) + 4 g + e % 4, whole 256-byte rows per instruction: streaming loads. rk[j], rv[j]
// cover group j from its first key's row at this KV head; a lane adds its fixed byte offsets:
// koff for K (key n, dims 8 g) and voff[i] for V (key 4 g + i, chunk n).
template <int D>
__device__ inline void load_k(KVFrag<D>& f, const __amdgpu_buffer_rsrc_t (&rk)[2], uint32_t koff) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int kk = 0; kk < KVFrag<D>::KSTEPS; ++kk)
      f.k[j][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk[j], koff + 64 * kk, 0, 0));
}
template <int D>
__device__ inline void load_v(KVFrag<D>& f, const __amdgpu_buffer_rsrc_t (&rv)[2],
                              const uint32_t (&voff)[4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (D == 128) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv[e >> 2], voff[e & 3], 0, kLoadStream);
      f.v[e][0] = x.x; f.v[e][1] = x.y; f.v[e][2] = x.z; f.v[e][3] = x.w;
    } else {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rv[e >> 2], voff[e & 3], 0, kLoadStream);
      f.v[e][0] = x.x; f.v[e][1] = x.y;
    }
  }
}

// One 32-key step: S^T = K Q^T, online softmax, O^T += V^T P^T. Two steps of loads stay in
// flight: the K registers take the loads of the step after next as soon as the score MFMAs have
// read them, the V registers as soon as the output MFMAs have (rk, rv: that step's groups).
// first_last_key: the smallest last visible key over the rows written out (wave-uniform); steps
// wholly below it and inside the range need no mask.
template <int D>
__device__ inline void compute_step(KVFrag<D>& f, const bf16x8 (&qf)[D / 32], int k0, int kend,
                                    int last_key, int first_last_key, float scale_log2, int g,
                                    float& m, float& l, f32x4 (&o)[D / 16],
                                    const __amdgpu_buffer_rsrc_t (&rk)[2],
                                    const __amdgpu_buffer_rsrc_t (&rv)[2], uint32_t koff,
                                    const uint32_t (&voff)[4]) {
  constexpr int KSTEPS = D / 32;
  f32x4 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) acc[j] = mfma16x16x32(f.k[j][kk], qf[kk], acc[j]);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_k<D>(f, rk, koff);
  const bool interior = k0 + 32 <= kend && k0 + 31 <= first_last_key;
  const bf16x8 pb =
      interior ? softmax_step<D / 16, false>(acc, k0, kend, last_key, scale_log2, g, m, l, o)
               : softmax_step<D / 16, true>(acc, k0, kend, last_key, scale_log2, g, m, l, o);
#pragma unroll
  for (int jt = 0; jt < D / 16; ++jt) o[jt] = mfma16x16x32(vt_operand<D>(f.v, jt), pb, o[jt]);
  __builtin_amdgcn_sched_barrier(0);
  load_v<D>(f, rv, voff);
}

// Block id of key k (uniform) from the partition's table entries held one per lane in three
// registers (entry jb0 + 64 r + lane in bt[r]). Each register is read with its own readlane and
// the result picked by a scalar select: indexing the array by jj would put it in memory.
__device__ inline int block_of(const int (&bt)[3], int jj) {
  const int l = jj & 63;
  const int b0 = __builtin_amdgcn_readlane(bt[0], l);
  const int b1 = __builtin_amdgcn_readlane(bt[1], l);
  const int b2 = __builtin_amdgcn_readlane(bt[2], l);
  return jj < 64 ? b0 : (jj < 128 ? b1 : b2);
}

// Small decode-only batches (at most 64 sequences, fewer (partition, KV head) items than waves)
// skip the planning launch: every wave derives the work list from the sequence inputs itself
// (one lane per sequence, the same validity rules and partition counts as the plan, a wave-wide
// scan) and takes the item that the first-round order across workgroups gives it; no queue. With
// the fused cache write, the waves left without an item write the step's K/V rows exactly as the
// write launch does, and each item's wave first writes the new rows inside its own partition at
// its KV head, then loads: the only rows of this step that an item reads are ones its own wave
// wrote (one wave's accesses to an address reach memory in issue order, and a fence keeps the
// compiler from moving the loads above the stores), so no wave waits for another. A row written
// twice gets the same bytes both times.
struct SelfPlan {
  WriteArgs w;  // w.k == nullptr: no cache write
  int32_t num_seqs, num_tokens, max_kv, max_blocks;
};

template <int D, bool SELF>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_kernel(
    const __bf16* __restrict__ q, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ block_tables,
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    __bf16* __restrict__ out, float* __restrict__ o_part, float* __restrict__ lse_part,
    const DecWork* __restrict__ items, const int32_t* __restrict__ counts,
    int32_t* __restrict__ queue, int32_t Hq, int32_t Hkv, BlockDiv bdiv,
    int32_t max_blocks_per_seq, int32_t P, int32_t max_splits, int32_t qmaxd,
    float scale_log2, SelfPlan sp) {
  constexpr int KSTEPS = D / 32;
  constexpr int NO = D / 16;  // output tiles (dims) per row
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int G = Hq / Hkv;
  const int bs = bdiv.bs;
  // self-planned, in the plan's order: every full partition (by sequence), then the sequences'
  // last partial partitions by decreasing length (the short ones land beside full ones when
  // workgroups take two). Lane s holds sequence s's inputs, its full partitions nf, the length
  // rm of its partial one (0: none), the inclusive scan of nf and the rank of its partial one.
  SeqIn sin{0, 0, 0};
  int nf = 0, rm = 0, incl = 0, rank = 0, nfull_all = 0;
  int total;
  if constexpr (SELF) {
    sin = seq_in(cu, kv_lens, lane, sp.num_seqs);
    int nfull, rem, np;
    const int ok = seq_items(sin, G, P, qmaxd, max_splits, 1, bs, sp.max_blocks, sp.max_kv, nfull,
                             rem, np);
    nf = ok && np == 0 ? nfull : 0;
    rm = ok && np == 0 ? rem : 0;
    incl = nf;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    nfull_all = __builtin_amdgcn_readlane(incl, 63);
    for (int t = 0; t < sp.num_seqs; ++t) {
      const int rt = __builtin_amdgcn_readlane(rm, t);
      rank += (rt > rm || (rt == rm && t < lane)) ? 1 : 0;
    }
    total = (nfull_all + (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(rm > 0))) * Hkv;
  } else {
    total = counts[0] * Hkv;
    // beside prefill work, only the first counts[4] workgroups (one per compute unit) take items
    if ((int)blockIdx.x >= counts[4]) return;
  }
  // per-lane byte offsets from a group's first cache row (see load_k, load_v)
  const uint32_t row_bytes = (uint32_t)Hkv * D * (uint32_t)sizeof(__bf16);
  const uint32_t koff = n * row_bytes + 16 * g;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (4 * g + i) * row_bytes + n * (D / 16) * (uint32_t)sizeof(__bf16);

  // Each wave takes (partition, KV head) items until they run out: every active wave first takes
  // one of items 0 .. nwaves - 1, then items nwaves + k for k = 0, 1, ... from the shared
  // counter, and leaves once its index passes `total`, so every item is taken once. The first
  // items need no atomic: all waves starting at once on one counter serialise. (Taking the next
  // index while the current item still streams was measured slower: near the end of the queue
  // it binds short items to waves that are still busy.) The first items go to the waves of a
  // workgroup in turn (the KV heads of a partition side by side on one CU, reading their
  // cache slots together), except when there are fewer items than waves: they are then dealt
  // across the workgroups, so that every CU streams (16 sequences of 256-2048 keys: 33.6 against
  // 45.0 us; from about 1.3 items per wave the grouped order is as fast or faster).
  const int wpb = (int)(blockDim.x >> 6);
  const int nblk = SELF ? (int)gridDim.x : min((int)gridDim.x, counts[4]);
  const int nwaves = nblk * wpb;
  const int wv = (int)(threadIdx.x >> 6);
  int idx = __builtin_amdgcn_readfirstlane(SELF || total < nwaves ? wv * nblk + (int)blockIdx.x
                                                                  : (int)blockIdx.x * wpb + wv);
  if constexpr (SELF) {
    // the host launches more waves than items: the rest write the step's K/V rows
    if (idx >= total) {
      if (sp.w.k)
        write_body(sp.w, cu, kv_lens, sp.num_seqs, sp.num_tokens, bs, sp.max_blocks, idx - total,
                   nwaves - total);
      return;
    }
  }
  for (;; ) {
    if (idx >= total) break;
    const int e = idx / Hkv;
    const int kvh = idx - e * Hkv;
    int s, split, q0, qn, L;
    if constexpr (SELF) {
      if (e < nfull_all) {  // full partition: the first lane whose inclusive count passes e
        s = __builtin_popcountll(__builtin_amdgcn_ballot_w64(incl <= e));
        split = e - (__builtin_amdgcn_readlane(incl, s) - __builtin_amdgcn_readlane(nf, s));
      } else {  // partial partition of rank e - nfull_all
        s = __builtin_ctzll(__builtin_amdgcn_ballot_w64(rm > 0 && rank == e - nfull_all));
        split = __builtin_amdgcn_readlane(nf, s);
      }
      q0 = __builtin_amdgcn_readlane(sin.c0, s);
      qn = __builtin_amdgcn_readlane(sin.q, s);
      L = __builtin_amdgcn_readlane(sin.L, s);
    } else {
      const DecWork w = items[e];
      s = w.seq;
      split = w.split;
      q0 = w.q0;
      qn = w.qn;
      L = w.L;
    }
    const int kb = split * P;
    const int ke = min(L, kb + P);
    const int nsplit = (L + P - 1) / P;
    const int rows = qn * G;

    // block-table entries of this partition, one per lane
    const int32_t* bt_row = block_tables + (int64_t)s * max_blocks_per_seq;
    const int jb0 = bdiv.div(kb);
    const int nbt = bdiv.div(ke + bs - 1) - jb0;
    // unconditional loads (indices clamped to the partition's last entry): no branch, no wait
    // between them
    int bt[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) bt[r] = bt_row[jb0 + min(64 * r + lane, nbt - 1)];

    // Q^T operand: lane column n is query row n = (token n / G, head n % G)
    // (loaded by every lane, from row 0 for the unused columns, then zeroed there: a branch
    // around the loads would make the first K/V loads wait for them)
    bf16x8 qf[KSTEPS];
    const bool qrow = n < rows;
    const int qi = qrow ? n / G : 0, hh = qrow ? n - (n / G) * G : 0;
    const int last_key = qrow ? L - qn + qi : -1;
    {
      const __bf16* pq = q + ((int64_t)(q0 + qi) * Hq + kvh * G + hh) * D + g * 8;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(pq + 32 * kk);
        qf[kk] = __builtin_bit_cast(bf16x8, qrow ? x : u32x4{0u, 0u, 0u, 0u});
      }
    }

    if constexpr (SELF) {
      // this step's new rows inside the partition, at this KV head (row p is token
      // q0 + p - (L - qn)), skipped where the slot mapping gives none; stored before any load
      if (sp.w.k) {
        constexpr int CPR = D / 8;    // 16-byte chunks of a row at one KV head
        constexpr int RPP = 64 / CPR;  // rows per pass of the wave
        const int c = lane % CPR;
        for (int p = max(kb, L - qn) + lane / CPR; p < ke; p += RPP) {
          const int j = bdiv.div(p);
          const int32_t blk = bt_row[j];
          const int64_t slot = (int64_t)blk * bs + (p - j * bs);
          if (blk >= 0 && slot < sp.w.slots) {
            const int64_t src = ((int64_t)(q0 + p - (L - qn)) * Hkv + kvh) * CPR + c;
            const int64_t dst = (slot * Hkv + kvh) * CPR + c;
            sp.w.k_cache[dst] = sp.w.k[src];
            sp.w.v_cache[dst] = sp.w.v[src];
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      }
    }

    float m = kMaxFloor, l = 0.f;
    f32x4 o[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int first_last_key = L - qn;  // last visible key of the item's first token

    // buffer resources of the two 16-key groups of the step starting at key k: the group's first
    // row at this KV head, records up to the range end (none for groups wholly past it)
    auto step_rsrc = [&](int k, __amdgpu_buffer_rsrc_t (&rk)[2], __amdgpu_buffer_rsrc_t (&rv)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int kg = k + 16 * j;
        const int kk = kg < ke ? kg : kb;
        const int bi = bdiv.div(kk);
        const int blk = block_of(bt, bi - jb0);
        const int64_t row = ((int64_t)(uint32_t)(blk * bs + (kk - bi * bs)) * Hkv + kvh) * D;
        const uint32_t nb = (uint32_t)min(max(ke - kg, 0), 16) * row_bytes;
        rk[j] = group_rsrc(k_cache + row, nb);
        rv[j] = group_rsrc(v_cache + row, nb);
      }
    };

    int k0 = kb;
    KVFrag<D> fa, fb;
    __amdgpu_buffer_rsrc_t rk[2], rv[2];
    step_rsrc(k0, rk, rv);
    load_k<D>(fa, rk, koff);
    load_v<D>(fa, rv, voff);
    step_rsrc(k0 + 32, rk, rv);
    load_k<D>(fb, rk, koff);
    load_v<D>(fb, rv, voff);
    // Steps go in pairs with one exit test per pair: a pair's second step past the range end is
    // fully masked (its loads read nothing and its probabilities are 0). An exit between the two
    // steps would let the compiler sink the first step's V loads past it, and the merged paths
    // make it wait for all loads at the top of the loop.
    do {
      step_rsrc(k0 + 64, rk, rv);
      compute_step<D>(fa, qf, k0, ke, last_key, first_last_key, scale_log2, g, m, l, o, rk, rv, koff, voff);
      step_rsrc(k0 + 96, rk, rv);
      compute_step<D>(fb, qf, k0 + 32, ke, last_key, first_last_key, scale_log2, g, m, l, o, rk, rv, koff, voff);
      k0 += 64;
    } while (k0 < ke);

    l = group_sum(l);  // the row's sum (all lanes take part)
    // lane (n, g) holds row n, dims (4g + i) * NO + jt
    if (n < rows) {
      const int qi = n / G, hh = n - (n / G) * G;
      const int h = kvh * G + hh;
      if (nsplit == 1) {
        const float inv = 1.f / l;
        __bf16* dst = out + ((int64_t)(q0 + qi) * Hq + h) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __bf16 r[NO];
#pragma unroll
          for (int jt = 0; jt < NO; ++jt) r[jt] = (__bf16)(o[jt][i] * inv);
          if constexpr (NO == 8)
            *reinterpret_cast<bf16x8*>(dst + (4 * g + i) * NO) = __builtin_bit_cast(bf16x8, r);
          else
            *reinterpret_cast<uint2*>(dst + (4 * g + i) * NO) = __builtin_bit_cast(uint2, r);
        }
      } else {
        const int64_t prow = (int64_t)s * qmaxd + qi;
        const int64_t base = (prow * Hq + h) * max_splits + split;
        const bool empty = !(l > 0.f);
        const float inv = empty ? 0.f : 1.f / l;
        float* dst = o_part + base * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float r[NO];
#pragma unroll
          for (int jt = 0; jt < NO; ++jt) r[jt] = o[jt][i] * inv;
#pragma unroll
          for (int c = 0; c < NO; c += 4)
            *reinterpret_cast<float4*>(dst + (4 * g + i) * NO + c) =
                make_float4(r[c], r[c + 1], r[c + 2], r[c + 3]);
        }
        if (g == 0) lse_part[base] = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
      }
    }
    if constexpr (SELF) break;  // every item is taken in the first round
    int next = 0;
    if (lane == 0) next = atomicAdd(queue, 1);
    idx = nwaves + __builtin_amdgcn_readfirstlane(next);
  }
}

// ---------------------------------------------------------------------------------------------
// 32 x 32 MFMA layout of the prefill kernel (v_mfma_f32_32x32x16_bf16). A operand: lane l holds
// row l % 32, contraction slots 8h .. 8h + 7 (h = l / 32); B operand: column l % 32, the same
// slots; C/D: column l % 32, rows 8(i / 4) + 4h + i % 4 for accumulator i = 0..15. The prefill
// kernel computes S^T = K Q^T (rows = 32 keys, columns = 32 query rows), so each lane holds 16
// of the 32 scores of its query row, the other 16 sitting in lane l ^ 32.

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum over lanes l and l ^ 32 (the two halves of a query row's scores)
__device__ inline float pair_max(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float pair_sum(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Online softmax over one 32-key chunk in the 32 x 32 layout: acc[i] is the score of key
// k0 + 8(i / 4) + 4h + i % 4 of this lane's row. Same scheme as chunk_max / rescale_lazy /
// chunk_exp: m is the row's reference max (scaled log2 units, equal in both lanes of the row),
// l this lane's part of the row sum.
template <bool MASK>
__device__ inline float chunk_max32(f32x16& acc, int k0, int kend, int last_key, float c, int h) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (MASK) {
      const int key = k0 + 8 * (i >> 2) + 4 * h + (i & 3);
      acc[i] = (key < kend && key <= last_key) ? acc[i] : -INFINITY;
    }
    mx = fmaxf(mx, acc[i]);
  }
  return mx * c;
}

template <int NDT>
__device__ inline void rescale_lazy32(float m_lane, float& m, float& l, f32x16 (&o)[NDT]) {
  if (__builtin_amdgcn_ballot_w64(m_lane > m + kRescaleSlack) != 0) {  // wave-uniform
    const float m_new = fmaxf(m, pair_max(m_lane));
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] *= alpha;
    m = m_new;
  }
}

// P^T operands of the chunk's two 16-key halves: slot e of half ks is key
// k0 + 16ks + 8(e / 4) + 4h + e % 4, i.e. accumulator 8ks + e.
// Adds a pair of bf16 probabilities to a row sum (one dot-product instruction against (1, 1)).
// The sum is taken over the bf16 values that the P V MFMAs multiply, so that the output's
// weights add up to one.
__device__ inline float add_pair(float s, __bf16 a, __bf16 b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 pr = {a, b}, one = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(pr, one, s, false);
}
__device__ inline void chunk_exp32(const f32x16& acc, float c, float m, float& l, bf16x8 (&pb)[2]) {
  float rs = 0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[ks][e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(acc[8 * ks + e], c, -m));
      if (e & 1) rs = add_pair(rs, pb[ks][e - 1], pb[ks][e]);
    }
  l += rs;
}

// ---------------------------------------------------------------------------------------------
// Prefill kernel: one workgroup of 8 waves (two per SIMD) per (query tile of 256 rows, KV head).
// Each wave owns 32 rows (one 32 x 32 MFMA tile). K/V tiles of 32 keys are gathered through the
// block table into LDS by all 512 threads and read by every wave. Three LDS tiles are in flight,
// so a wave can overlap its matrix and vector work: while the exponentials of tile t run on the
// VALU, the S^T = K Q^T products of tile t + 1 run on the matrix cores, and the P V products of
// tile t run beside the row maxima of tile t + 1. A step starts by storing tile t + 2 (loaded
// into registers two steps earlier) to LDS and loading tile t + 4 into the registers it frees.
// The scale stays in fp32, applied to each score beside its exponential: scaling Q before the
// MFMAs would round c q to bf16, a relative error of 2^-9 on every product q_i k_i, which for
// keys of large magnitude moves the logits by hundredths of a log2 unit (measured: outputs off
// by up to 0.06 on keys growing to 11x, against 0.015 with the scale in fp32).

constexpr int kPrefillKeys = 32;  // keys per LDS tile (one barrier per tile)
constexpr int kPrefillBufs = 3;   // LDS tiles: being computed, ready, being filled

template <int D>
struct PrefillSmem {
  // bf16 per LDS row. LDS serves 64 banks of 4 bytes (256 bytes per clock). A K fragment read
  // takes 16 bytes from each of 16 consecutive rows per 16 lanes served together: rows 304
  // bytes apart (D = 128) or 144 (D = 64) put those at 16 distinct bank groups. A V^T
  // transposing read takes 64 bytes from each of 4 consecutive rows per 32 lanes: rows
  // 2D + 64 bytes apart put the four runs on distinct quarters of the banks. Measured on
  // the 70B-shaped chunks: V rows 304 bytes apart cost 6.6e7 bank-conflict cycles per launch
  // (29% of the LDS's busy cycles), 320 bytes apart none.
  static constexpr int STRIDE = D == 128 ? D + 24 : D + 8;
  static constexpr int VSTRIDE = D + 32;
  __bf16 k[kPrefillBufs][kPrefillKeys][STRIDE];
  __bf16 v[kPrefillBufs][kPrefillKeys][VSTRIDE];
};

template <int D>
__global__ __launch_bounds__(kPrefillWaves * 64)
__attribute__((amdgpu_waves_per_eu(kPrefillWavesPerSimd, kPrefillWavesPerSimd)))
void prefill_kernel(
    const __bf16* __restrict__ q, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ block_tables,
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    __bf16* __restrict__ out, const Work* __restrict__ items, const int32_t* __restrict__ counts,
    float* __restrict__ o_pre, float* __restrict__ lse_pre, int32_t* __restrict__ nsplit_tok,
    int32_t maxs, int32_t Hq, int32_t Hkv, BlockDiv bdiv, int32_t max_blocks_per_seq, int32_t bq,
    float scale_log2) {
  constexpr int KS = kPrefillKeys;
  const int bs = bdiv.bs;
  constexpr int KK = D / 16;   // 32x32x16 MFMA k-steps over the head dimension
  constexpr int NDT = D / 32;  // 32-dim output tiles
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
  // threads that load K/V (a whole number of waves) and key rows they cover per pass
  constexpr int LOADERS = kPrefillWaves * 64 < KS * CPR ? kPrefillWaves * 64 : KS * CPR;
  constexpr int RPP = LOADERS / CPR;
  constexpr int PASSES = KS / RPP;
  static_assert(RPP % 16 == 0 && KS % RPP == 0 && LOADERS % 64 == 0,
                "a load pass must cover whole 16-key groups");
  using SmemT = PrefillSmem<D>;
  __shared__ __attribute__((aligned(16))) SmemT sm;

  const int item = blockIdx.x / Hkv;
  const int kvh = blockIdx.x - item * Hkv;
  // the item count and the item's record in one round trip (items has room for every workgroup
  // of the grid); workgroups past the count leave
  const int n_items = counts[1];
  const Work w = items[item];
  if (item >= n_items) return;
  const int s = w.seq, qt = w.idx / kMaxPreSplits, part = w.idx - qt * kMaxPreSplits;
  const int G = Hq / Hkv;
  const int q0 = w.q0;
  const int qn = w.qn;
  const int L = w.L;
  const int tok0 = qt * bq;
  const int tok_end = min(qn, tok0 + bq);
  // keys [0, kend_tile) are visible to some row of the tile; this part covers [kb, kend)
  const int kend_tile = L - qn + tok_end;
  int ns, chunk;
  prefill_split(kend_tile, counts[3] ? maxs : 1, ns, chunk);
  const int kb = part * chunk;  // a multiple of KS
  const int kend = min(kend_tile, kb + chunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, h = lane >> 5;  // this lane's query row of the wave, row half

  // Q^T operand (B of S^T = K Q^T): lane l holds dims [16kk + 8h, +8) of query row
  // R = 32 wave + l % 32, row = (token R / G, head R % G)
  bf16x8 qf[KK];
  int last_key;
  {
    const int R = wave * 32 + n32;
    const int qi = tok0 + R / G, hh = R - (R / G) * G;
    if (qi < tok_end) {
      const __bf16* p = q + ((int64_t)(q0 + qi) * Hq + kvh * G + hh) * D + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(p + 16 * kk);
      last_key = L - qn + qi;
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.f;
      last_key = -1;
    }
  }

  // smallest last visible key over this wave's rows (its first row's token); rows past tok_end
  // have zero Q, finite scores and are never written
  const int wave_first_last_key = L - qn + tok0 + wave * 32 / G;

  // Loader role of this thread: key row lr + pass * RPP of each tile, 16-byte chunk lc. A pass
  // covers whole 16-key groups, each inside one block, so the block id and in-block offset of a
  // group are wave-uniform; only the row within the group is per lane. When the tile has fewer
  // chunks than the workgroup has threads, the extra threads repeat the first ones (same loads,
  // same LDS stores), so that every wave runs the same load pipeline.
  const int ltid = LOADERS < kPrefillWaves * 64 ? tid % LOADERS : tid;
  const int lr = ltid / CPR, lc = ltid - (ltid / CPR) * CPR;
  const int32_t* bt_row = block_tables + (int64_t)s * max_blocks_per_seq;
  // The group of a pass that a lane loads is lr / 16 = ltid / (16 CPR): whole waves share it, so
  // a group's cache address is a scalar and each lane adds a fixed byte offset (row within the
  // group, chunk).
  static_assert((16 * CPR) % 64 == 0 && LOADERS % (16 * CPR) == 0, "load groups are wave-uniform");
  const int lane_grp = __builtin_amdgcn_readfirstlane(lr >> 4);
  const uint32_t lane_off = ((lr & 15) * Hkv * D + lc * 8) * (uint32_t)sizeof(__bf16);
  const int64_t row_elems = (int64_t)Hkv * D;  // elements per cache row (token slot)
  const uint32_t row_bytes = (uint32_t)(Hkv * D * sizeof(__bf16));
  const __bf16* k_head = k_cache + (int64_t)kvh * D;
  const __bf16* v_head = v_cache + (int64_t)kvh * D;
  auto blk_of = [&](int key) __attribute__((always_inline)) { return bdiv.div(key); };
  // Block ids come from a window of the sequence's block-table row held in one register: lane i
  // has the entry of block w0 + i. A group's id is read with readlane (no memory wait in the
  // steps); the window moves (one vector load, waited on) once per 64 blocks.
  const int nbt = bdiv.div(kend + bs - 1);  // table entries the part reads
  int w0 = bdiv.div(kb);
  int win = w0 + lane < nbt ? bt_row[w0 + lane] : 0;
  asm volatile("" : : "v"(win));
  // keep the blocks of tile `step` inside the window (tiles are visited in increasing order)
  auto slide_window = [&](int step) __attribute__((always_inline)) {
    const int k_last = min(kb + step * KS + KS, kend) - 1;
    if (blk_of(k_last) >= w0 + 64) {  // wave-uniform
      w0 = blk_of(kb + step * KS);
      win = w0 + lane < nbt ? bt_row[w0 + lane] : 0;
      // consume the load here, so that no wait for it is left to the reads in every step
      asm volatile("" : : "v"(win));
    }
  };
  // Two register sets stage tile loads: tile t goes through set t % 2. A step first stores its
  // set to LDS and then reloads that set with the tile two steps on, so the loads of a tile have
  // two whole steps to arrive. Every step loads and stores a tile (past the last tile, the last
  // one again, into a buffer nobody reads), so the number of loads in flight is the same on
  // every path.
  uint4 rk[2][PASSES], rv[2][PASSES];
  // Load tile `step` into register set X, each 16-key group through a buffer descriptor whose
  // record count ends at kend (groups wholly past it keep the tile's first group as their base
  // and read nothing).
  auto fetch = [&](auto set_tag, int step) __attribute__((always_inline)) {
    constexpr int X = decltype(set_tag)::value;
    slide_window(step);
    const int t0 = kb + step * KS;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int kg = t0 + ps * RPP + 16 * lane_grp;
      const int key = kg < kend ? kg : t0;
      const int bi = blk_of(key);
      const int blk = __builtin_amdgcn_readlane(win, bi - w0);
      const int64_t row = (int64_t)(uint32_t)(blk * bs + (key - bi * bs)) * row_elems;
      // records: the group's rows before kend (a max and a select, which stay scalar: a clamp
      // becomes a vector median instruction); rows at or past kend load as zeros
      const int rem = kend - kg;
      const uint32_t nb = rem >= 16 ? 0xffffffffu : (uint32_t)max(rem, 0) * row_bytes;
      rk[X][ps] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(group_rsrc(k_head + row, nb), lane_off, 0, 0));
      rv[X][ps] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(group_rsrc(v_head + row, nb), lane_off, 0, 0));
    }
  };
  // Store register set X to LDS buffer buf. Rows at or past kend hold zeros (their
  // loads read nothing), so that a masked probability (0) never meets an unwritten V value.
  auto stash = [&](auto set_tag, int buf) __attribute__((always_inline)) {
    constexpr int X = decltype(set_tag)::value;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      *reinterpret_cast<uint4*>(&sm.k[buf][lr + ps * RPP][lc * 8]) = rk[X][ps];
      *reinterpret_cast<uint4*>(&sm.v[buf][lr + ps * RPP][lc * 8]) = rv[X][ps];
    }
  };

  // S^T = K Q^T of LDS tile `buf`: A = K rows (lane l: key l % 32, dims [16kk + 8h, +8))
  auto qk = [&](int buf, f32x16& acc) __attribute__((always_inline)) {
    acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sm.k[buf][n32][16 * kk + 8 * h]);
      acc = mfma32x32x16(kf, qf[kk], acc);
    }
  };
  // O^T += V^T P^T of LDS tile `buf`, per 32-dim tile dt and 16-key half ks. The V^T operand
  // (A: lane l holds dim 32dt + l % 32 for the slots of P^T's half ks) comes from transposing
  // LDS reads: within each 16-lane group, lanes 4j + a read key 16ks + 8e' + 4h + j, dims
  // 32dt + 16(group % 2) + 4a .. +3, and lane 4a + b receives element b of the four reads: dim
  // 32dt + l % 32, keys 16ks + 8e' + 4h + j, j = 0..3 (slots 4e' + j).
  f32x16 o[NDT];
  auto pv = [&](int buf, const bf16x8 (&pb)[2]) __attribute__((always_inline)) {
    const int r = lane & 15;
    const __bf16* vb = &sm.v[buf][4 * h + (r >> 2)][16 * ((lane >> 4) & 1) + 4 * (r & 3)];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const s16x4 lo = lds_read_tr16(vb + (16 * ks) * SmemT::VSTRIDE + 32 * dt);
        const s16x4 hi = lds_read_tr16(vb + (16 * ks + 8) * SmemT::VSTRIDE + 32 * dt);
        const bf16x8 vt =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = mfma32x32x16(vt, pb[ks], o[dt]);
      }
  };

  float m = kMaxFloor, l = 0.f;
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x16{};

  // Tiles whose keys are all visible to every row of this wave take no mask; the rest (the
  // causal diagonal and the range end) do. The split differs between waves, but every wave runs
  // the same steps, so the barriers pair up in order.
  const int nsteps = (kend - kb + KS - 1) / KS;  // >= 1
  const int n_open = min(nsteps, max(0, min(kend, wave_first_last_key + 1) - kb) / KS);

  // The two waves of a SIMD run half a step apart: a step is an issue-bound half (score MFMAs
  // with the exponentials) and an MFMA-bound half (output MFMAs with the max), and group A runs
  // them in that order before the step's barrier while group B passes the barrier between them,
  // so that one wave's first half meets the other's second half. The group is the wave's rank
  // among the waves of its SIMD (hardware id register), exchanged through LDS.
  __shared__ int wave_simd[kPrefillWaves];
  const int my_simd = __builtin_amdgcn_readfirstlane(
      (int)__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4));  // HW_ID bits 5:4 (SIMD)
  if (lane == 0) wave_simd[wave] = my_simd;

  // prologue: tiles 0 and 1 into LDS, tiles 2 and 3 into register sets 0 and 1 (tile indices
  // past the last tile stand for the last tile)
  const int last_tile = nsteps - 1;
  fetch(Int<0>{}, 0);
  fetch(Int<1>{}, min(1, last_tile));
  stash(Int<0>{}, 0);
  stash(Int<1>{}, 1);
  fetch(Int<0>{}, min(2, last_tile));
  fetch(Int<1>{}, min(3, last_tile));
  __syncthreads();
  int grp = 0;
  for (int w = 0; w < wave; ++w) grp |= wave_simd[w] == my_simd;
  grp = __builtin_amdgcn_readfirstlane(grp);

  // scores of even tiles live in accA, of odd tiles in accB (no copy between steps)
  f32x16 accA, accB;
  qk(0, accA);
  {
    const float mc = n_open > 0 ? chunk_max32<false>(accA, kb, kend, last_key, scale_log2, h)
                                : chunk_max32<true>(accA, kb, kend, last_key, scale_log2, h);
    rescale_lazy32<NDT>(mc, m, l, o);
  }

  // step st < nsteps - 1: tile st is in LDS buffer cur with its scores (masked) in accA / accB
  // by the parity P = st % 2 and its reference max settled; tile st + 1 is in buffer nxt; buffer
  // fil receives tile st + 2 from register set P, which then receives tile st + 4.
  // The order of the work is fixed with scheduling barriers: the K fragments of tile st + 1 are
  // read first; each of the KK score MFMAs of tile st + 1 then follows VPP V^T reads of tile st;
  // each of the 2 NDT output MFMAs of tile st carries part of the max of tile st + 1. The
  // exponentials of tile st are written beside the score MFMAs, but the compiler sinks them past
  // the mid-step barrier to the start of the second half, next to the output MFMAs that use
  // them; with the two waves of a SIMD half a step apart, one wave's exponentials then meet the
  // other's score MFMAs. Measured on 70B-shaped chunks: pinning them under the same wave's score
  // MFMAs is 8% slower (1.17 vs 1.08 ms), and so is one wave per SIMD with two row tiles each.
  constexpr int EPP = 16 / KK;
  constexpr int VPP = 4 * NDT / KK;
  constexpr int XPP = 16 / (2 * NDT);
  static_assert(16 % KK == 0 && (4 * NDT) % KK == 0 && 16 % (2 * NDT) == 0, "step layout");
  int cur = 0, nxt = 1, fil = 2;
  // carried from the first half of a step to the second: V^T fragments and probabilities of
  // tile st (the second half's operands)
  s16x4 vr[4 * NDT];
  bf16x8 pb[2];
  auto half1 = [&](auto parity_tag, int st) __attribute__((always_inline)) {
    constexpr int P = decltype(parity_tag)::value;
    const f32x16& acc = P ? accB : accA;
    f32x16& acc_n = P ? accA : accB;
    bf16x8 kf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(&sm.k[nxt][n32][16 * kk + 8 * h]);
    stash(Int<P>{}, fil);
    fetch(Int<P>{}, min(st + 4, last_tile));
    __builtin_amdgcn_sched_barrier(0);
    // V^T read j of tile st: key half ks = j / (2 NDT), dim tile dt = (j / 2) % NDT, 8-key half
    // j % 2 (the operand layout of pv above)
    const int r = lane & 15;
    const __bf16* vb = &sm.v[cur][4 * h + (r >> 2)][16 * ((lane >> 4) & 1) + 4 * (r & 3)];
    float rs = 0.f;
    acc_n = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const int i = kk * EPP + e;
        pb[i / 8][i % 8] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], scale_log2, -m));
        if (e & 1) rs = add_pair(rs, pb[i / 8][i % 8 - 1], pb[i / 8][i % 8]);
      }
#pragma unroll
      for (int v = 0; v < VPP; ++v) {
        const int j = kk * VPP + v;
        vr[j] = lds_read_tr16(vb + (16 * (j / (2 * NDT)) + 8 * (j % 2)) * SmemT::VSTRIDE +
                              32 * ((j / 2) % NDT));
      }
      acc_n = mfma32x32x16(kf[kk], qf[kk], acc_n);
      __builtin_amdgcn_sched_barrier(0);
    }
    l += rs;
  };
  auto half2 = [&](auto mask_tag, auto parity_tag, int st) __attribute__((always_inline)) {
    constexpr bool MASK_NEXT = decltype(mask_tag)::value;
    constexpr int P = decltype(parity_tag)::value;
    f32x16& acc_n = P ? accA : accB;
    float mx = -INFINITY;
    const int k0n = kb + (st + 1) * KS;
    // this half is MFMA-bound: its MFMAs go first when both waves of the SIMD are ready, so the
    // other wave's exponentials fill the gaps (measured 0.5-1% faster than equal priority)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int pc = 0; pc < 2 * NDT; ++pc) {
      const int ks = pc / NDT, dt = pc % NDT, j = ks * 2 * NDT + 2 * dt;
      const bf16x8 vt =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(vr[j], vr[j + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = mfma32x32x16(vt, pb[ks], o[dt]);
#pragma unroll
      for (int e = 0; e < XPP; ++e) {
        const int i = pc * XPP + e;
        if (MASK_NEXT) {
          const int key = k0n + 8 * (i >> 2) + 4 * h + (i & 3);
          acc_n[i] = (key < kend && key <= last_key) ? acc_n[i] : -INFINITY;
        }
        mx = fmaxf(mx, acc_n[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    const float mc = mx * scale_log2;
    rescale_lazy32<NDT>(mc, m, l, o);
    const int t = cur;
    cur = nxt;
    nxt = fil;
    fil = t;
  };
  // one barrier per step for every wave: group B's between the halves, group A's after them
  auto step = [&](auto mask_tag, auto parity_tag, int st) __attribute__((always_inline)) {
    half1(parity_tag, st);
    if (grp) __syncthreads();
    half2(mask_tag, parity_tag, st);
    if (!grp) __syncthreads();
  };
  // steps [st, end) with the register-set parity known at compile time
  int st = 0;
  auto run = [&](auto mask_tag, int end) __attribute__((always_inline)) {
    if ((st & 1) && st < end) step(mask_tag, Int<1>{}, st++);
    for (; st + 1 < end; st += 2) {
      step(mask_tag, Int<0>{}, st);
      step(mask_tag, Int<1>{}, st + 1);
    }
    if (st < end) step(mask_tag, Int<0>{}, st++);
  };
  run(Tag<false>{}, n_open - 1);
  run(Tag<true>{}, nsteps - 1);
  {
    const f32x16 acc_last = (nsteps - 1) & 1 ? accB : accA;
    bf16x8 pb[2];
    chunk_exp32(acc_last, scale_log2, m, l, pb);
    pv(cur, pb);
  }

  l = pair_sum(l);  // the row's sum (all lanes take part)
  if (ns > 1 && part == 0 && kvh == 0)  // the merge finds this tile's tokens by their count
    for (int i = tid; i < tok_end - tok0; i += kPrefillWaves * 64) nsplit_tok[q0 + tok0 + i] = ns;
  // normalise and store: lane l holds query row R = 32 wave + l % 32, dims
  // 32dt + 8(i / 4) + 4h + i % 4 of tile dt; a part of a split tile stores fp32 o and its lse
  {
    const int R = wave * 32 + n32;
    const int qi = tok0 + R / G, hh = R - (R / G) * G;
    if (qi < tok_end) {
      const int64_t row = (int64_t)(q0 + qi) * Hq + kvh * G + hh;
      if (ns > 1) {
        const bool empty = !(l > 0.f);  // no visible key in this part
        const float inv = empty ? 0.f : 1.f / l;
        const int64_t pb = row * maxs + part;
        float* dst = o_pre + pb * D + 4 * h;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4*>(dst + 32 * dt + 8 * g4) =
                make_float4(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv, o[dt][4 * g4 + 2] * inv,
                            o[dt][4 * g4 + 3] * inv);
        if (h == 0) lse_pre[pb] = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
      } else {
        const float inv = 1.f / l;
        __bf16* dst = out + row * D + 4 * h;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            __bf16 r4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r4[i] = (__bf16)(o[dt][4 * g4 + i] * inv);
            *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * g4) = __builtin_bit_cast(uint2, r4);
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Log-sum-exp merge of KV partitions. GS adjacent threads per (partial row, head, 8-dim chunk):
// thread pg of the group takes partitions pg, pg + GS, ..., and the group combines its maxima and
// sums with lane shuffles. GS = kReduceGroup when rows may have more than 4 batches of partitions
// (a long row's partitions are then read with a quarter of the round trips per thread: 8.2
// against 18.8 us for 16 long-context rows of up to 128 partitions), else 1: for many rows of few
// partitions the extra threads and their first loads only cost (at 256 sequences of up to 4
// partitions 11.5 against 5.3 us, at 128 of up to 16 14.9 against 9.0).
// INTERNAL: partial row = (sequence, token of the sequence), count derived from kv_lens.
// Otherwise: partial row = packed token, count from num_splits.
// A thread's first kReduceBatch partitions' lse and o are loaded together with the count (slots
// past the count are read but never used), so a typical row costs one memory round trip; later
// ones 16 at a time.
constexpr int kReduceGroup = 4;
constexpr int kReduceBatch = 8;

template <int N>
__device__ inline void merge_accumulate(const float4 (&a)[N], const float4 (&b)[N],
                                        const float (&lk)[N], int kmax, float M,
                                        float& wsum, float (&acc)[8]) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    // an empty partition (lse = -inf) has no weight and its o is never used
    if (k < kmax && lk[k] != -INFINITY) {
      const float wk = __builtin_amdgcn_exp2f((lk[k] - M) * kLog2e);
      wsum += wk;
      acc[0] += wk * a[k].x; acc[1] += wk * a[k].y; acc[2] += wk * a[k].z; acc[3] += wk * a[k].w;
      acc[4] += wk * b[k].x; acc[5] += wk * b[k].y; acc[6] += wk * b[k].z; acc[7] += wk * b[k].w;
    }
  }
}

// entries of a strided list below ns: partitions first, first + GS, ... < ns
template <int GS>
__device__ inline int strided_count(int ns, int first) {
  return ns > first ? (ns - first + GS - 1) / GS : 0;
}

// MODE: kReduceStandalone (cb_split_kv_reduce: split count per token from the caller),
// kReduceDecode (decode rows of the attention call: count from the sequence's length),
// kReducePrefill (tokens of split prefill tiles: count written by the prefill kernel; a token
// with a count below 2 was written directly and is skipped before any partial is read).
enum { kReduceStandalone = 0, kReduceDecode = 1, kReducePrefill = 2 };

// gid: GS * (row-head-chunk index) + pg. Every early return depends on the row only, so the
// threads of a group return together or reach the shuffles together.
template <int D, int MODE, int GS>
__device__ inline void merge_one(int64_t gid, const float* __restrict__ o_part,
                                 const float* __restrict__ lse_part,
                                 const int32_t* __restrict__ num_splits, __bf16* __restrict__ out,
                                 int32_t Hq, int32_t max_splits, int64_t nrows,
                                 const int32_t* __restrict__ cu, const int32_t* __restrict__ kv_lens,
                                 int32_t qmaxd, int32_t G, int32_t P) {
  constexpr int CH = D / 8;
  const int pg = (int)(gid % GS);
  const int64_t x = gid / GS;
  const int64_t per_row = (int64_t)Hq * CH;
  const int64_t prow = x / per_row;
  if (prow >= nrows) return;
  const int rem = (int)(x - prow * per_row);
  const int h = rem / CH, c = rem - (rem / CH) * CH;
  const int64_t base = (prow * Hq + h) * max_splits;
  int ns_pre = 0;
  if constexpr (MODE == kReducePrefill) {
    ns_pre = min(num_splits[prow], max_splits);
    if (ns_pre < 2) return;
  }
  const int lim = MODE == kReducePrefill ? ns_pre : max_splits;  // partitions that may be read
  float lk[kReduceBatch];
  float4 a[kReduceBatch], b[kReduceBatch];
#pragma unroll
  for (int i = 0; i < kReduceBatch; ++i) {
    const int k = pg + GS * i;
    lk[i] = -INFINITY;
    if (k < lim) {
      lk[i] = lse_part[base + k];
      const float4* p = reinterpret_cast<const float4*>(o_part + (base + k) * D + c * 8);
      a[i] = p[0];
      b[i] = p[1];
    }
  }
  int64_t t;
  int ns;
  if constexpr (MODE == kReduceDecode) {
    const int s = (int)(prow / qmaxd), qi = (int)(prow - (prow / qmaxd) * qmaxd);
    const int qn = cu[s + 1] - cu[s];
    if (qi >= qn || qn * G > 16 || qn > qmaxd) return;
    ns = (kv_lens[s] + P - 1) / P;
    if (ns <= 1 || ns > max_splits) return;  // single partition: written directly
    t = cu[s] + qi;
  } else if constexpr (MODE == kReducePrefill) {
    t = prow;
    ns = ns_pre;
  } else {
    t = prow;
    ns = min(num_splits[t], max_splits);
    if (ns <= 0) return;
  }
  constexpr int first_rest = GS * kReduceBatch;  // partitions of the up-front loads
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kReduceBatch; ++i)
    if (pg + GS * i < ns) M = fmaxf(M, lk[i]);
  for (int k0 = pg + first_rest; k0 < ns; k0 += GS * 16) {
    float xm[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) xm[j] = k0 + GS * j < ns ? lse_part[base + k0 + GS * j] : -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) M = fmaxf(M, xm[j]);
  }
#pragma unroll
  for (int m = 1; m < GS; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {  // the same in the whole group
    merge_accumulate(a, b, lk, strided_count<GS>(ns, pg), M, wsum, acc);
    for (int k0 = pg + first_rest; k0 < ns; k0 += GS * 16) {
      float lx[16];
      float4 ax[16], bx[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int k = k0 + GS * j;
        lx[j] = -INFINITY;
        if (k < ns) {
          lx[j] = lse_part[base + k];
          const float4* p = reinterpret_cast<const float4*>(o_part + (base + k) * D + c * 8);
          ax[j] = p[0];
          bx[j] = p[1];
        }
      }
      merge_accumulate(ax, bx, lx, strided_count<GS>(ns, k0), M, wsum, acc);
    }
  }
#pragma unroll
  for (int m = 1; m < GS; m <<= 1) {
    wsum += __shfl_xor(wsum, m, 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], m, 64);
  }
  if (pg != 0) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  __bf16 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x8*>(out + (t * Hq + h) * D + c * 8) = __builtin_bit_cast(bf16x8, r);
}

// GS threads per (row, head, 8-dim chunk); the prefill merge strides over all tokens with a
// small grid, since most tokens (those of unsplit tiles and of decodes) only read their count.
template <int D, int MODE, int GS>
__global__ __launch_bounds__(256) void reduce_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const int32_t* __restrict__ num_splits, __bf16* __restrict__ out, int32_t Hq,
    int32_t max_splits, int64_t nrows, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ kv_lens, int32_t qmaxd, int32_t G, int32_t P,
    const int32_t* __restrict__ split_flag) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if constexpr (MODE == kReducePrefill) {
    if (*split_flag == 0) return;  // the plan split no prefill tile
    const int64_t total = nrows * Hq * (D / 8) * GS;
    for (int64_t x = gid; x < total; x += (int64_t)gridDim.x * 256)
      merge_one<D, MODE, GS>(x, o_part, lse_part, num_splits, out, Hq, max_splits, nrows, cu,
                             kv_lens, qmaxd, G, P);
  } else {
    merge_one<D, MODE, GS>(gid, o_part, lse_part, num_splits, out, Hq, max_splits, nrows, cu,
                           kv_lens, qmaxd, G, P);
  }
}

// ---------------------------------------------------------------------------------------------
// Host side

// Launch of the decode-row or standalone merge over `rows` partial rows: groups of kReduceGroup
// threads per (row, head, chunk) when a row may have more than 4 batches of partitions, else one.
// Returns false when the grid would exceed the launch limit.
template <int MODE>
bool launch_merge(int head_dim, int64_t rows, int32_t Hq, int32_t max_splits, hipStream_t st,
                  const float* o_part, const float* lse_part, const int32_t* num_splits,
                  __bf16* out, const int32_t* cu, const int32_t* kv_lens, int32_t qmaxd,
                  int32_t G, int32_t P) {
  const bool grouped = max_splits > 4 * kReduceBatch;
  const int64_t threads = rows * Hq * (head_dim / 8) * (grouped ? kReduceGroup : 1);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return false;
  const unsigned g = (unsigned)grid;
  if (head_dim == 128) {
    if (grouped)
      reduce_kernel<128, MODE, kReduceGroup><<<g, 256, 0, st>>>(o_part, lse_part, num_splits, out, Hq,
          max_splits, rows, cu, kv_lens, qmaxd, G, P, nullptr);
    else
      reduce_kernel<128, MODE, 1><<<g, 256, 0, st>>>(o_part, lse_part, num_splits, out, Hq, max_splits,
          rows, cu, kv_lens, qmaxd, G, P, nullptr);
  } else {
    if (grouped)
      reduce_kernel<64, MODE, kReduceGroup><<<g, 256, 0, st>>>(o_part, lse_part, num_splits, out, Hq,
          max_splits, rows, cu, kv_lens, qmaxd, G, P, nullptr);
    else
      reduce_kernel<64, MODE, 1><<<g, 256, 0, st>>>(o_part, lse_part, num_splits, out, Hq, max_splits,
          rows, cu, kv_lens, qmaxd, G, P, nullptr);
  }
  return true;
}

struct Plan {
  int32_t G = 0, P = 0, max_splits = 0, qmaxd = 0, bq = 0, pre_splits = 1;
  int64_t dec_cap = 0, pre_cap = 0;
  size_t off_counts = 0, off_dec = 0, off_pre = 0, off_opart = 0, off_lse = 0;
  size_t off_opre = 0, off_lsepre = 0, off_nsplit = 0, total = 0;
};

// Prefill partials take num_tokens * Hq * pre_splits * (D + 1) fp32 of workspace; splitting is
// offered only while that stays within this budget.
constexpr size_t kPrefillPartialBudget = size_t(256) << 20;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Scratch of the no-allocation entry point (cb_paged_attention_write_noalloc): device memory the
// library holds for the life of the process, one copy per device, in place of a caller
// workspace. 128 MiB holds the decode partials of every workload measured here (the largest,
// 131 sequences of up to 16K keys with 64 query heads, needs 69 MB); prefill partials are held
// to a quarter of it (tiles whose partials would need more are not split along the keys).
constexpr size_t kNoAllocScratchBytes = CB_NOALLOC_SCRATCH_BYTES;
constexpr size_t kNoAllocPrefillBudget = kNoAllocScratchBytes / 4;

int32_t choose_split(int32_t num_seqs, int32_t Hkv, int32_t max_kv_len, int32_t requested,
                     bool decode_only) {
  if (requested > 0) {
    int32_t p = (int32_t)cb::ceil_div(requested, 32) * 32;
    return p > kMaxSplitTokens ? kMaxSplitTokens : p;
  }
  // About 5461 (partition, KV head) items over the batch's upper-bound key count, in steps of 256
  // keys: 8/3 per wave of a decode launch on 256 CUs (2048 waves), about 4/3 per wave for
  // uniformly drawn lengths. Measured on decode-only batches (several draws each), this picked
  // the fastest size or one within 5% of it: 1536 at 256 sequences of up to 4K keys (a
  // power-of-two rule's 1024 was 4-8% slower), 768 at 64 of up to 8K, 2048 at 16 of up to 128K,
  // and 2048 against 1536's 5% better at 128 of up to 16K (the 2048 cap). The same rule holds
  // beside prefill work: over four draws of the 8B-shaped mixed 2048-token batch its 768 took
  // the fused step 0.6-3% less time than partitions 1.5 times larger.
  // Below that rule's 256-key floor a decode-only batch has too few keys to fill the launch
  // with balanced items, and the size trades other costs: shorter partitions spread a small
  // batch's keys over more waves, longer ones pay fewer item starts (each several memory round
  // trips) and fewer partials to merge. Measured on 34 draws of 1-120 sequences of up to 700 to
  // 131072 keys (fused step, 8B-shaped heads, sizes 128-2048), the fastest size tracked about
  // one 640th of the upper-bound keys (at least a 24th of the longest sequence), but no more
  // than 768 unless the longest sequence is over 8 times that (a few long sequences stream best
  // in long items); one partition per sequence (no merge) won wherever it needed at most twice
  // that size. This choice came within 1.8% of the fastest measured size on average (8.5% at
  // worst).
  const int64_t keys = (int64_t)max_kv_len * num_seqs * Hkv;
  const int64_t p = (keys / 5461 + 128) / 256 * 256;
  if (decode_only && p <= 256) {
    const int64_t L = max_kv_len;
    int64_t d = std::max<int64_t>((keys + 639) / 640, (L + 23) / 24);
    d = std::min<int64_t>(d, std::max<int64_t>(768, L / 8));
    d = std::min<int64_t>(kMaxSplitTokens, std::max<int64_t>(128, (d + 63) / 64 * 64));
    if (2 * d >= L) d = std::max<int64_t>(32, (L + 31) / 32 * 32);
    return (int32_t)d;
  }
  return (int32_t)std::min<int64_t>(kMaxSplitTokens, std::max<int64_t>(256, p));
}

Plan make_plan(int32_t num_seqs, int32_t num_tokens, int32_t Hq, int32_t Hkv, int32_t D,
               int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens,
               size_t pre_budget = kPrefillPartialBudget) {
  Plan p;
  p.G = Hq / Hkv;
  const int32_t dec_q = 16 / p.G;  // longest decode-type chunk
  p.P = choose_split(num_seqs, Hkv, max_kv_len, kv_split_tokens, (int64_t)max_q_len * p.G <= 16);
  p.max_splits = (int32_t)cb::ceil_div(max_kv_len, p.P);
  p.qmaxd = max_q_len < dec_q ? max_q_len : dec_q;
  p.bq = kPrefillRows / p.G;
  p.dec_cap = (int64_t)num_seqs * p.max_splits;
  if (max_q_len > dec_q) {
    const size_t per_split = (size_t)num_tokens * Hq * (D + 1) * sizeof(float);
    const size_t fit = per_split > 0 ? pre_budget / per_split : 0;
    p.pre_splits = (int32_t)std::min<size_t>(kMaxPreSplits, std::max<size_t>(1, fit));
    if (p.pre_splits < 2) p.pre_splits = 1;
  }
  p.pre_cap = (max_q_len > dec_q) ? ((int64_t)num_tokens / p.bq + num_seqs) * p.pre_splits : 0;
  size_t off = 0;
  p.off_counts = off;
  off = align256(off + 32);
  p.off_dec = off;
  off = align256(off + sizeof(DecWork) * (size_t)p.dec_cap);
  p.off_pre = off;
  off = align256(off + sizeof(Work) * (size_t)p.pre_cap);
  const size_t nrows = p.max_splits > 1 ? (size_t)num_seqs * p.qmaxd * Hq * p.max_splits : 0;
  p.off_opart = off;
  off = align256(off + sizeof(float) * nrows * D);
  p.off_lse = off;
  off = align256(off + sizeof(float) * nrows);
  const size_t prows = p.pre_splits > 1 ? (size_t)num_tokens * Hq * p.pre_splits : 0;
  p.off_opre = off;
  off = align256(off + sizeof(float) * prows * D);
  p.off_lsepre = off;
  off = align256(off + sizeof(float) * prows);
  p.off_nsplit = off;
  off = align256(off + (p.pre_splits > 1 ? sizeof(int32_t) * (size_t)num_tokens : 0));
  p.total = off;
  return p;
}

bool supported_ratio(int32_t G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

// Compute units of the current device, queried once per device.
bool device_cus(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return true;
    }
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
    return false;
  if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  *out = v;
  return true;
}

// Second stream for the decode kernel, so that it runs beside the prefill kernel (the one is
// HBM-bound, the other MFMA-bound): one per (device, caller stream), created on first use, kept
// until the process ends, default priority. fork / join order it after the planning kernel and
// before the merge on the caller's stream. At most kMaxAuxStreams caller streams per device get
// one; calls on further caller streams run the decode kernel after the prefill kernel on the
// caller's stream instead (same results, no overlap), so the table stays bounded however many
// streams a caller cycles through.
//
// Host threads that enqueue on one caller stream at the same time share its fork and join
// events. Each call records an event and makes the other stream wait on it right away, so a
// wait always covers at least that call's own work (it may also cover another thread's work
// enqueued in between: extra ordering, never missing ordering).
constexpr int kMaxAuxStreams = 64;

struct AuxStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

enum class Aux { kOk, kFull, kError };

Aux aux_stream(hipStream_t st, AuxStream* out) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, AuxStream> table;
  static int per_device[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Aux::kError;
  std::lock_guard<std::mutex> lock(mu);
  auto it = table.find({dev, st});
  if (it != table.end()) {
    *out = it->second;
    return Aux::kOk;
  }
  if (dev < 0 || dev >= 64 || per_device[dev] >= kMaxAuxStreams) return Aux::kFull;
  AuxStream a;
  if (hipStreamCreateWithFlags(&a.stream, hipStreamNonBlocking) != hipSuccess) return Aux::kError;
  if (hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess)
    return Aux::kError;
  table[{dev, st}] = a;
  ++per_device[dev];
  *out = a;
  return Aux::kOk;
}

}  // namespace

extern "C" int32_t cb_paged_attention_split_tokens(int32_t num_seqs, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t max_q_len,
                                                   int32_t max_kv_len, int32_t kv_split_tokens) {
  const int32_t G = num_kv_heads > 0 && num_q_heads >= num_kv_heads ? num_q_heads / num_kv_heads : 1;
  return choose_split(num_seqs, num_kv_heads, max_kv_len, kv_split_tokens,
                      (int64_t)max_q_len * G <= 16);
}

extern "C" size_t cb_paged_attention_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                                    int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_dim, int32_t block_size,
                                                    int32_t max_q_len, int32_t max_kv_len,
                                                    int32_t kv_split_tokens) {
  (void)block_size;
  if (num_seqs <= 0 || num_tokens <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      max_q_len <= 0 || max_kv_len <= 0)
    return 0;
  return make_plan(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_q_len,
                   max_kv_len, kv_split_tokens < 0 ? 0 : kv_split_tokens)
      .total;
}

namespace {
// pending request of cb_time_next_kernel (per thread, one-shot)
struct KernelTimer {
  int which = 0;
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local KernelTimer g_timer;

bool record_if(const KernelTimer& tm, int which, bool start, hipStream_t st) {
  if (tm.which != which) return true;
  return hipEventRecord(start ? tm.start : tm.stop, st) == hipSuccess;
}
}  // namespace

extern "C" int cb_time_next_kernel(int32_t which, void* start_event, void* stop_event) {
  using cb::fail;
  if (which != 0 && which != CB_KERNEL_DECODE && which != CB_KERNEL_PREFILL)
    return fail(CB_ERR_INVALID_ARG, "cb_time_next_kernel: unknown kernel id " + std::to_string(which));
  if (which != 0 && (!start_event || !stop_event))
    return fail(CB_ERR_INVALID_ARG, "cb_time_next_kernel: NULL event");
  g_timer = KernelTimer{which, static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return cb::ok();
}

namespace {

// The no-allocation entry point's scratch. In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, once per device, and
// only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up on the first call per device).
bool scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return false;
    addr[dev] = p;
  }
  *out = addr[dev];
  return true;
}

}  // namespace

namespace {

// cb_paged_attention, and with k_new / v_new given, cb_paged_attention_write (the cache write
// runs beside the planning workgroup in the first launch).
int attention_impl(const void* q_packed, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                   const int32_t* block_tables, const void* k_cache, const void* v_cache, void* out,
                   float scale, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_q_len,
                   int32_t max_kv_len, int32_t kv_split_tokens, void* workspace,
                   size_t workspace_bytes, void* stream, const void* k_new, const void* v_new,
                   bool no_alloc = false) {
  using cb::fail;
  const int E = CB_ERR_INVALID_ARG;
  const KernelTimer tm = g_timer;  // one-shot: consumed by this call
  g_timer = KernelTimer{};
  if (block_size < 4) return fail(E, "block_size must be at least 4, got " + std::to_string(block_size));
  if (num_seqs < 0 || num_tokens < 0) return fail(E, "negative num_seqs or num_tokens");
  if (num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1) return fail(E, "head counts and head_dim must be positive");
  if (num_q_heads % num_kv_heads != 0) return fail(E, "num_q_heads must be a multiple of num_kv_heads");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(E, "scale must be finite and positive");
  if (kv_split_tokens < 0) return fail(E, "kv_split_tokens must be >= 0");
  if (head_dim != 64 && head_dim != 128) return fail(CB_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!supported_ratio(num_q_heads / num_kv_heads))
    return fail(CB_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads must be 1, 2, 4, 8 or 16");
  if (block_size % 16 != 0) return fail(CB_ERR_UNSUPPORTED, "block_size must be a multiple of 16");
  if (num_seqs == 0 || num_tokens == 0) return cb::ok();
  if (!q_packed || !cu_seqlens_q || !kv_lens || !block_tables || !k_cache || !v_cache || !out)
    return fail(E, "cb_paged_attention: NULL pointer argument");
  if (!cb::aligned16(q_packed) || !cb::aligned16(k_cache) || !cb::aligned16(v_cache) || !cb::aligned16(out))
    return fail(E, "q_packed, caches and out must be 16-byte aligned");
  if (max_blocks_per_seq < 1 || num_blocks < 1) return fail(E, "max_blocks_per_seq and num_blocks must be >= 1");
  if (max_q_len < 1 || max_kv_len < 1) return fail(E, "max_q_len and max_kv_len must be >= 1");
  if (max_kv_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(E, "max_kv_len exceeds the block-table capacity max_blocks_per_seq * block_size");
  const Plan p = make_plan(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_q_len,
                           max_kv_len, kv_split_tokens,
                           no_alloc ? kNoAllocPrefillBudget : kPrefillPartialBudget);
  if (no_alloc) {
    if (p.total > kNoAllocScratchBytes)
      return fail(CB_ERR_WORKSPACE, "cb_paged_attention_write_noalloc: this batch needs " +
                                        std::to_string(p.total) + " bytes of scratch, more than the " +
                                        std::to_string(kNoAllocScratchBytes) + " the library holds");
    if (!scratch_address(&workspace))
      return fail(CB_ERR_HIP, "cb_paged_attention_write_noalloc: hipGetSymbolAddress(scratch) failed");
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || workspace_bytes < p.total)
    return fail(CB_ERR_WORKSPACE, "workspace needs " + std::to_string(p.total) + " bytes, got " +
                                      std::to_string(workspace_bytes));
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(E, "workspace must be 256-byte aligned");
  if ((int64_t)p.dec_cap * num_kv_heads > INT32_MAX || (int64_t)p.pre_cap * num_kv_heads > INT32_MAX)
    return fail(CB_ERR_UNSUPPORTED, "batch too large for one launch");

  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.off_counts);
  DecWork* dec = reinterpret_cast<DecWork*>(ws + p.off_dec);
  Work* pre = reinterpret_cast<Work*>(ws + p.off_pre);
  float* o_part = reinterpret_cast<float*>(ws + p.off_opart);
  float* lse_part = reinterpret_cast<float*>(ws + p.off_lse);
  float* o_pre = reinterpret_cast<float*>(ws + p.off_opre);
  float* lse_pre = reinterpret_cast<float*>(ws + p.off_lsepre);
  int32_t* nsplit_tok = reinterpret_cast<int32_t*>(ws + p.off_nsplit);
  int cus = 0;
  if (!device_cus(&cus)) return fail(CB_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
  const float scale_log2 = scale * kLog2e;
  const __bf16* qp = static_cast<const __bf16*>(q_packed);
  const __bf16* kc = static_cast<const __bf16*>(k_cache);
  const __bf16* vc = static_cast<const __bf16*>(v_cache);
  __bf16* op = static_cast<__bf16*>(out);

  // With prefill work, the decode kernel goes to the second stream and overlaps the prefill
  // (not in the no-allocation variant, which creates no stream, nor on a caller stream past the
  // per-device limit: there it follows the prefill kernel on the caller's stream, with the whole
  // GPU). The plan sizes the decode kernel's share of the compute units accordingly.
  hipStream_t dst = st;
  AuxStream aux;
  if (p.pre_cap > 0 && p.dec_cap > 0 && !no_alloc) {
    const Aux a = aux_stream(st, &aux);
    if (a == Aux::kError) return fail(CB_ERR_HIP, "creating the decode stream failed");
    if (a == Aux::kOk) dst = aux.stream;
  }
  const int32_t beside = dst != st ? 1 : 0;

  WriteArgs w{};
  if (k_new)
    w = WriteArgs{static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                  static_cast<uint4*>(const_cast<void*>(k_cache)), static_cast<uint4*>(const_cast<void*>(v_cache)),
                  block_tables, (int32_t)((int64_t)num_kv_heads * head_dim * 2 / 16),
                  num_blocks * block_size};
  // A decode-only batch of at most 64 sequences whose (partition, KV head) items stay below the
  // waves of two 4-wave workgroups per compute unit plans itself inside the decode kernel (see
  // SelfPlan): no planning launch.
  const bool self_plan = p.pre_cap == 0 && num_seqs >= 1 && num_seqs <= 64 &&
                         p.dec_cap * num_kv_heads < 2LL * (kDecodeWaves / 2) * cus;
  if (!self_plan && k_new) {
    // one wave per token, 16 waves per workgroup
    const int64_t nw = std::min<int64_t>(cb::ceil_div(num_tokens, 16), 4 * (int64_t)cus);
    plan_write_kernel<<<(unsigned)(1 + nw), 1024, 0, st>>>(
        cu_seqlens_q, kv_lens, num_seqs, p.G, p.P, p.qmaxd, p.max_splits, p.bq, block_size,
        max_blocks_per_seq, max_kv_len, dec, p.dec_cap, pre, p.pre_cap, counts, num_kv_heads, cus,
        p.pre_splits, num_tokens, 4 * head_dim, nsplit_tok, beside, w);
  } else if (!self_plan) {
    plan_kernel<<<1, 1024, 0, st>>>(cu_seqlens_q, kv_lens, num_seqs, p.G, p.P, p.qmaxd,
                                    p.max_splits, p.bq, block_size, max_blocks_per_seq, max_kv_len, dec,
                                    p.dec_cap, pre, p.pre_cap, counts, num_kv_heads, cus, p.pre_splits,
                                    num_tokens, 4 * head_dim, nsplit_tok, beside);
  }
  if (dst != st) {
    if (hipEventRecord(aux.fork, st) != hipSuccess || hipStreamWaitEvent(aux.stream, aux.fork, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "decode stream fork failed");
  }
  if (p.pre_cap > 0) {
    // one workgroup per (item, KV head); workgroups past the plan's item count exit at once.
    // Tiles are split only while tiles * Hkv < 2 * CUs, so items * Hkv stays below
    // 2 * CUs * pre_splits then, which bounds the grid beside the unsplit tile bound.
    const int64_t unsplit = p.pre_cap / p.pre_splits * num_kv_heads;
    const int64_t grid64 = std::min<int64_t>(
        p.pre_cap * num_kv_heads,
        p.pre_splits > 1 ? std::max<int64_t>(unsplit, 2 * (int64_t)cus * p.pre_splits) : unsplit);
    const unsigned grid = (unsigned)grid64;
    if (!record_if(tm, CB_KERNEL_PREFILL, true, st)) return fail(CB_ERR_HIP, "hipEventRecord failed");
    if (head_dim == 128)
      prefill_kernel<128><<<grid, kPrefillWaves * 64, 0, st>>>(
          qp, cu_seqlens_q, kv_lens, block_tables, kc, vc, op, pre, counts, o_pre, lse_pre,
          nsplit_tok, p.pre_splits, num_q_heads, num_kv_heads, block_div(block_size),
          max_blocks_per_seq, p.bq, scale_log2);
    else
      prefill_kernel<64><<<grid, kPrefillWaves * 64, 0, st>>>(
          qp, cu_seqlens_q, kv_lens, block_tables, kc, vc, op, pre, counts, o_pre, lse_pre,
          nsplit_tok, p.pre_splits, num_q_heads, num_kv_heads, block_div(block_size),
          max_blocks_per_seq, p.bq, scale_log2);
    if (!record_if(tm, CB_KERNEL_PREFILL, false, st)) return fail(CB_ERR_HIP, "hipEventRecord failed");
    // merge the parts of split prefill tiles (tokens of other tiles skip); no tile can split
    // when no sequence is longer than one part
    if (p.pre_splits > 1 && max_kv_len > kPrefillSplitKeys) {
      const int64_t threads = (int64_t)num_tokens * num_q_heads * (head_dim / 8);
      const unsigned mgrid = (unsigned)std::min<int64_t>((threads + 255) / 256, 2 * (int64_t)cus);
      if (head_dim == 128)
        reduce_kernel<128, kReducePrefill, 1><<<mgrid, 256, 0, st>>>(
            o_pre, lse_pre, nsplit_tok, op, num_q_heads, p.pre_splits, num_tokens, nullptr,
            nullptr, 0, 0, 0, counts + 3);
      else
        reduce_kernel<64, kReducePrefill, 1><<<mgrid, 256, 0, st>>>(
            o_pre, lse_pre, nsplit_tok, op, num_q_heads, p.pre_splits, num_tokens, nullptr,
            nullptr, 0, 0, 0, counts + 3);
    }
  }
  {
    // Persistent, 2 waves per SIMD. Beside prefill work: one 8-wave workgroup per compute unit
    // (the whole register file, so a compute unit holds either decode or prefill work and none is
    // left over), of which the plan lets counts[4] work; never more waves than items. Otherwise
    // 4-wave workgroups, one or two per compute unit for every unit: a batch with fewer items
    // than waves has them dealt across the workgroups, and a grid between one and two per unit
    // would give some units twice the others' share (measured on 22 small decode-only batches:
    // up to 15% less time with whole rounds, never more than 2% more).
    // (self-planned: at least one wave more than items, for the cache write)
    const int64_t items = p.dec_cap * num_kv_heads + (self_plan ? 1 : 0);
    const int waves = dst != st ? kDecodeWaves : kDecodeWaves / 2;
    const int64_t per_cu = dst != st ? 1 : 2;
    int64_t groups = std::max<int64_t>(1, std::min<int64_t>((items + waves - 1) / waves, per_cu * (int64_t)cus));
    if (dst == st) groups = std::min<int64_t>(per_cu * (int64_t)cus, (groups + cus - 1) / cus * cus);
    const unsigned grid = (unsigned)groups;
    int32_t* queue = counts + 2;
    if (!record_if(tm, CB_KERNEL_DECODE, true, dst)) return fail(CB_ERR_HIP, "hipEventRecord failed");
    const SelfPlan sp{w, num_seqs, num_tokens, max_kv_len, max_blocks_per_seq};
    const BlockDiv bdiv = block_div(block_size);
#define CB_DECODE_LAUNCH(DIM, SELF_)                                                             \
  decode_kernel<DIM, SELF_><<<grid, waves * 64, 0, dst>>>(                                       \
      qp, cu_seqlens_q, kv_lens, block_tables, kc, vc, op, o_part, lse_part, dec, counts, queue, \
      num_q_heads, num_kv_heads, bdiv, max_blocks_per_seq, p.P, p.max_splits, p.qmaxd,          \
      scale_log2, sp)
    if (head_dim == 128) {
      if (self_plan) CB_DECODE_LAUNCH(128, true); else CB_DECODE_LAUNCH(128, false);
    } else {
      if (self_plan) CB_DECODE_LAUNCH(64, true); else CB_DECODE_LAUNCH(64, false);
    }
#undef CB_DECODE_LAUNCH
    if (!record_if(tm, CB_KERNEL_DECODE, false, dst)) return fail(CB_ERR_HIP, "hipEventRecord failed");
  }
  if (dst != st) {
    if (hipEventRecord(aux.join, dst) != hipSuccess || hipStreamWaitEvent(st, aux.join, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "decode stream join failed");
  }
  if (p.max_splits > 1) {
    const int64_t nrows = (int64_t)num_seqs * p.qmaxd;
    if (!launch_merge<kReduceDecode>(head_dim, nrows, num_q_heads, p.max_splits, st, o_part,
                                     lse_part, nullptr, op, cu_seqlens_q, kv_lens, p.qmaxd, p.G,
                                     p.P))
      return fail(CB_ERR_UNSUPPORTED, "batch too large for one merge launch");
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CB_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return cb::ok();
}

}  // namespace

extern "C" int cb_paged_attention(const void* q_packed, const int32_t* cu_seqlens_q,
                                  const int32_t* kv_lens, const int32_t* block_tables,
                                  const void* k_cache, const void* v_cache, void* out, float scale,
                                  int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(q_packed, cu_seqlens_q, kv_lens, block_tables, k_cache, v_cache, out, scale,
                        num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, max_q_len, max_kv_len, kv_split_tokens,
                        workspace, workspace_bytes, stream, nullptr, nullptr);
}

extern "C" int cb_paged_attention_write(const void* q_packed, const void* k_new, const void* v_new,
                                        const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                        const int32_t* block_tables, void* k_cache, void* v_cache,
                                        void* out, float scale, int32_t num_seqs, int32_t num_tokens,
                                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_blocks_per_seq,
                                        int64_t num_blocks, int32_t max_q_len, int32_t max_kv_len,
                                        int32_t kv_split_tokens, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && num_tokens > 0) {
    if (!k_new || !v_new) return cb::fail(CB_ERR_INVALID_ARG, "cb_paged_attention_write: NULL k_new or v_new");
    if (!cb::aligned16(k_new) || !cb::aligned16(v_new))
      return cb::fail(CB_ERR_INVALID_ARG, "cb_paged_attention_write: k_new and v_new must be 16-byte aligned");
    if (num_blocks > 0 && block_size > 0 && num_blocks * (int64_t)block_size > INT32_MAX)
      return cb::fail(CB_ERR_INVALID_ARG, "num_blocks * block_size must stay below 2^31");
  }
  return attention_impl(q_packed, cu_seqlens_q, kv_lens, block_tables, k_cache, v_cache, out, scale,
                        num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, max_q_len, max_kv_len, kv_split_tokens,
                        workspace, workspace_bytes, stream, k_new ? k_new : nullptr, v_new);
}


extern "C" int cb_paged_attention_write_noalloc(
    const void* q_packed, const void* k_new, const void* v_new, const int32_t* cu_seqlens_q,
    const int32_t* kv_lens, const int32_t* block_tables, void* k_cache, void* v_cache, void* out,
    float scale, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens, void* stream) {
  if (num_seqs > 0 && num_tokens > 0) {
    if (!k_new || !v_new)
      return cb::fail(CB_ERR_INVALID_ARG, "cb_paged_attention_write_noalloc: NULL k_new or v_new");
    if (!cb::aligned16(k_new) || !cb::aligned16(v_new))
      return cb::fail(CB_ERR_INVALID_ARG,
                      "cb_paged_attention_write_noalloc: k_new and v_new must be 16-byte aligned");
    if (num_blocks > 0 && block_size > 0 && num_blocks * (int64_t)block_size > INT32_MAX)
      return cb::fail(CB_ERR_INVALID_ARG, "num_blocks * block_size must stay below 2^31");
  }
  return attention_impl(q_packed, cu_seqlens_q, kv_lens, block_tables, k_cache, v_cache, out, scale,
                        num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, max_q_len, max_kv_len, kv_split_tokens,
                        nullptr, 0, stream, k_new, v_new, /*no_alloc=*/true);
}

extern "C" int cb_split_kv_reduce(const float* o_part, const float* lse_part,
                                  const int32_t* num_splits, void* out, int32_t num_tokens,
                                  int32_t num_q_heads, int32_t head_dim, int32_t max_splits,
                                  void* stream) {
  using cb::fail;
  if (num_tokens < 0 || num_q_heads < 1 || max_splits < 1)
    return fail(CB_ERR_INVALID_ARG, "cb_split_kv_reduce: bad size argument");
  if (head_dim != 64 && head_dim != 128) return fail(CB_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_tokens == 0) return cb::ok();
  if (!o_part || !lse_part || !num_splits || !out)
    return fail(CB_ERR_INVALID_ARG, "cb_split_kv_reduce: NULL pointer argument");
  if (!cb::aligned16(o_part) || !cb::aligned16(out))
    return fail(CB_ERR_INVALID_ARG, "o_part and out must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  __bf16* op = static_cast<__bf16*>(out);
  if (!launch_merge<kReduceStandalone>(head_dim, num_tokens, num_q_heads, max_splits, st, o_part,
                                       lse_part, num_splits, op, nullptr, nullptr, 1, 1, 1))
    return fail(CB_ERR_UNSUPPORTED, "cb_split_kv_reduce: too many rows");
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CB_ERR_HIP, std::string("reduce launch: ") + hipGetErrorString(e));
  return cb::ok();
}
