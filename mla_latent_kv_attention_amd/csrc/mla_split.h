// mla_split.h -- pieces of the split-KV decode shared by the decode and verify kernels:
// the batch's step list (each sequence's key range cut into 16-token steps, laid end to
// end and divided into equal pieces), the lse merge of a sequence's shares by its last
// piece, and work-group reductions over the sequences.
#pragma once

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla_impl {
namespace {

using namespace mla_dev;

constexpr int kStep = 16;  // tokens per step of the step list

// Dims held by lane group `grp` for k-step kk of the 576-wide contraction: a
// pair of k-steps covers 16 consecutive dims per lane (one 16-byte load of fp8
// codes, two of bf16).  The same map is used for keys and queries, so any
// permutation of the contraction index is fine.
__device__ __forceinline__ int kdim(int kk, int grp) {
  return 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1);
}

// Four consecutive output values of row n, fp32 or bf16.
__device__ __forceinline__ void store_row4(const DecodeParams& p, size_t n, int d, f32x4 v) {
  if (p.out_bf16) {
    const bf16x4 o = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    *(bf16x4*)((uint16_t*)p.out + n * kDV + d) = o;
  } else {
    *(f32x4*)((float*)p.out + n * kDV + d) = v;
  }
}

// int32 in the constant address space: a uniform index reads it with a scalar load.
typedef __attribute__((address_space(4))) const int32_t kconst_i32;

// Key range of sequence b this call covers, in 16-token steps from `base`.
struct SeqRange {
  int L, lo, hi, base, n;
};

// Row rr of sequence b in q, out and lse (this launch's rows sit at r_off in each sequence).
__device__ __forceinline__ size_t io_row(const DecodeParams& p, int b, int rr) {
  return (size_t)b * p.r_stride + p.r_off + rr;
}

// The sequence length as this launch sees it: a group of positions that ends
// len_shift positions before the sequence's last keeps the same causal limits
// (position j sees keys < L - P + j + 1) with L and P taken as the group's.
__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int b) {
  SeqRange r;
  r.L = ((const kconst_i32*)p.seq_lens)[b] - p.len_shift;
  r.lo = p.kv_begin ? max(((const kconst_i32*)p.kv_begin)[b], 0) : 0;
  r.hi = p.kv_end ? min(((const kconst_i32*)p.kv_end)[b], r.L) : r.L;
  r.base = r.lo & ~(kStep - 1);
  r.n = r.hi > r.lo ? (r.hi - r.base + kStep - 1) / kStep : 0;
  return r;
}

// a / b for non-negative a, b > 0: 32-bit when both fit (the usual case), which
// is far shorter than the 64-bit division sequence.
__device__ __forceinline__ long div_nonneg(long a, long b) {
  if (((unsigned long)(a | b) >> 32) == 0) return (long)((uint32_t)a / (uint32_t)b);
  return a / b;
}

// Work-group w of W owns steps [first_step(w), first_step(w + 1)) of the batch's
// concatenated step list; step s belongs to owner(s).
__device__ __forceinline__ long first_step(long w, long N, int W) { return div_nonneg(w * N, W); }
__device__ __forceinline__ int owner(long s, long N, int W) {
  return (int)div_nonneg((s + 1) * W - 1, N);
}

// Last piece of sequence b: combine the partials of pieces w_first..w_last for
// row rr (16 threads per row, 4 dims each per 64-dim slab).  The pieces are taken
// four at a time, each batch's lse values loaded together with its partial rows,
// and combined online against a running maximum (one global round trip per batch,
// none for a separate pass over the lse values).  A piece that saw no key of the
// row has lse = -inf and an unwritten row, which its zero weight selects away.
__device__ __forceinline__ void merge_pieces(const DecodeParams& p, int b, int rr, size_t n,
                                             int w_first, int w_last) {
  const int j = threadIdx.x & 15;
  const size_t R = p.R;
  const float* lse_b = p.part_lse + (size_t)b * R + rr;  // slot v at v * R
  // slot v's rows start at part_out + (v + b) * R * 512; this lane's bytes within it
  const uint32_t off = (uint32_t)(rr * kDV + 4 * j) * 4;
  float mx = -INFINITY, ls = 0.f;
  f32x4 o8[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o8[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int v0 = w_first; v0 <= w_last; v0 += 4) {
    float l4[4];
    f32x4 x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = min(v0 + u, w_last);  // past the end: re-read the last slot, weight 0
      l4[u] = (v0 + u <= w_last) ? load_agent(lse_b + v * R) : -INFINITY;
      const auto rsrc = agent_rsrc(p.part_out + (size_t)(v + b) * R * kDV);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[u][k] = load_agent16(rsrc, off + 256 * k);
    }
    const float m_new = fmaxf(fmaxf(mx, fmaxf(l4[0], l4[1])), fmaxf(l4[2], l4[3]));
    if (m_new == -INFINITY) continue;  // nothing seen yet
    const float r = (mx == -INFINITY) ? 0.f : expf(mx - m_new);
    ls *= r;
#pragma unroll
    for (int k = 0; k < 8; ++k) o8[k] *= r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wt = (l4[u] == -INFINITY) ? 0.f : expf(l4[u] - m_new);
      ls += wt;
      if (wt > 0.f)
#pragma unroll
        for (int k = 0; k < 8; ++k) o8[k] += wt * x[u][k];
    }
    mx = m_new;
  }
  if (mx != -INFINITY) {
    const float il = 1.f / ls;
#pragma unroll
    for (int k = 0; k < 8; ++k) o8[k] *= il;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) store_row4(p, n, 4 * j + 64 * k, o8[k]);
  if (p.lse && j == 0) p.lse[n] = (mx == -INFINITY) ? -INFINITY : mx + logf(ls);
}

// Error flags (MLA_FLAG_* in mla.h): bits ORed into the workspace's flags word.
constexpr int kFlagStaleCounters = 1;
constexpr int kFlagBadLengths = 2;
constexpr int kFlagBadBlocks = 4;

__device__ __forceinline__ void raise_flag(const DecodeParams& p, int bit) {
  if (p.flags) __hip_atomic_fetch_or(p.flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Piece 0's check of sequence b's lengths against the stated contract (P <= seq_lens <=
// max_blocks * block_size, kv_begin >= 0); results are undefined outside it.
__device__ __forceinline__ void check_lengths(const DecodeParams& p, int b) {
  const int L = p.seq_lens[b] - p.len_shift;
  const bool bad = L < p.P || (long)L > (long)p.max_blocks * p.block_size ||
                   (p.kv_begin && p.kv_begin[b] < 0);
  if (bad) raise_flag(p, kFlagBadLengths);
}

// Physical block of logical block i in a sequence's block-table row bt (a uniform
// index: the id comes through the scalar cache).  A negative id, outside the
// contract, would address memory before the cache: block 0 is read instead, and the
// ids are OR-ed into `seen`, whose sign bit the caller checks to flag the call once its
// loop is done (a branch here would make every block-id load wait at once).
__device__ __forceinline__ long block_id(const kconst_i32* bt, int i, int& seen) {
  const int id = bt[i];
  seen |= id;
  return id < 0 ? 0 : id;
}

// The same with the flag raised at once.  (In the bf16 decode kernel the deferred
// form above changes the register allocation enough to spill; there this one is
// kept.)
__device__ __forceinline__ long block_id_now(const DecodeParams& p, const kconst_i32* bt, int i) {
  const int id = bt[i];
  if (id < 0) {
    raise_flag(p, kFlagBadBlocks);
    return 0;
  }
  return id;
}

// Sum over the work-group (256 threads); sh holds 4 values and is free on entry.
__device__ __forceinline__ long long block_sum(long long v, long long* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  const long long t = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return t;
}

// Exclusive prefix sum over the work-group in thread order; *total gets the sum.
__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* sh,
                                                          long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  long long before = 0;
  for (int i = 0; i < wave; ++i) before += sh[i];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return before + incl - v;
}


}  // namespace
}  // namespace mla_impl
