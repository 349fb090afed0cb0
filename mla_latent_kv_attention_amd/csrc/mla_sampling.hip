// mla_sampling.hip -- top-k renormalisation of probability rows for gfx950.
//
// The acceptance step after a speculative verify needs the target distribution
// cut to its k most likely tokens: keep the k largest entries of each row, set
// the rest to zero and rescale the kept ones to sum to one (tahou.com article,
// section "ROCm适配迎来突破，软件壁垒不再高不可攀"; 66bd.net article, section
// "我们是如何做到的").  Exactly k entries are kept; entries rank by value in IEEE
// total order (-0 below +0, a positive NaN above +inf) and, among equal values,
// the lower index first; k <= 0 or k >= vocab keeps the whole row; a kept sum of
// zero gives a zero row.
//
// The op is HBM-bound: read the row once, write it once.  Two launches:
//  1. one 512-thread work-group per 16,384-entry chunk of a row holds its chunk
//     in registers (32 entries per thread), finds the chunk's k-th largest entry
//     by a radix select on order-preserving 32-bit keys (digits of 11, 11 and 10
//     bits, counted in an LDS histogram), writes the chunk's k candidates (key,
//     index) in index order to the workspace and zero-fills its output range.
//     The row's top k are among the union of its chunks' top k.
//  2. one 1024-thread work-group per row selects the row's k-th largest among
//     its candidates the same way, resolves ties at the threshold by a second
//     select on the index, sums the kept entries in a fixed order and writes
//     p / sum over the kept positions.
// For k above kListMax (or a chunk shorter than k) a chunk keeps no list: the
// second launch reads that chunk's entries straight from the input.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla_impl {
using namespace mla_dev;

namespace {

constexpr int kT1 = 512;                       // first-stage threads
constexpr int kRounds = 8;                     // float4 loads per first-stage thread
constexpr int kChunk = kRounds * 4 * kT1;      // 16,384 entries per chunk
constexpr int kT2 = 1024;                      // second-stage threads
constexpr int kHistBins = 2048;

// Order-preserving map of an fp32 value to uint32 and back.
__device__ __forceinline__ uint32_t rank_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Radix-select digit passes: bits [21, 32), [10, 21), [0, 10).
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int digit_bins(int pass) { return pass == 2 ? 1024 : 2048; }

// Inclusive prefix sum over the work-group in thread order; *total gets the sum.
// wsum holds NT / 64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t w = wsum[i];
    before += (i < wv) ? w : 0u;
    tot += w;
  }
  __syncthreads();
  *total = tot;
  return before + v;
}

// The same for four independent sums at once.  wsum holds 4 * NT / 64 words.
template <int NT>
__device__ __forceinline__ u32x4 block_incl_scan4(u32x4 v, uint32_t* wsum, u32x4* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    u32x4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = __shfl_up(v[q], o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) *(u32x4*)(wsum + 4 * wv) = v;
  __syncthreads();
  u32x4 before = {0u, 0u, 0u, 0u}, tot = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const u32x4 w = *(const u32x4*)(wsum + 4 * i);
    if (i < wv) before += w;
    tot += w;
  }
  __syncthreads();
  *total = tot;
  return before + v;
}

// Sum over the work-group in a fixed order (so the result is the same on every run).
template <int NT>
__device__ __forceinline__ float block_sum_f32(float v, float* wsum) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += wsum[i];
  __syncthreads();
  return t;
}

// hist[0..nbins) counts entries per digit.  Finds the digit d holding the rem-th
// largest counted entry (entries above d < rem <= entries above d + hist[d]) and
// writes d and the count above it to sel[0], sel[1].  Needs 1 <= rem <= total.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nbins, uint32_t rem,
                                           uint32_t* wsum, uint32_t* sel) {
  const int per = nbins / NT;  // bins per thread: 1, 2 or 4
  const int b0 = threadIdx.x * per;
  uint32_t s = 0;
  for (int i = 0; i < per; ++i) s += hist[b0 + i];
  uint32_t tot;
  const uint32_t incl = block_incl_scan<NT>(s, wsum, &tot);
  uint32_t above = tot - incl;  // entries in the bins above this thread's range
  for (int i = per - 1; i >= 0; --i) {
    const uint32_t h = hist[b0 + i];
    if (above < rem && rem <= above + h) {
      sel[0] = (uint32_t)(b0 + i);
      sel[1] = above;
    }
    above += h;
  }
  __syncthreads();
}

// The row's kept count: k <= 0 or k >= vocab keeps all of it.
__device__ __forceinline__ int kept_count(int k, int vocab) {
  return (k <= 0 || k >= vocab) ? vocab : k;
}

// A chunk of len entries keeps a candidate list iff k < len and k <= list_max.
__device__ __forceinline__ bool has_list(int keff, int len, int list_max) {
  return keff < len && keff <= list_max;
}

template <bool kVec>
__global__ __launch_bounds__(kT1) void topk_chunk_kernel(const float* __restrict__ probs,
                                                         const int32_t* __restrict__ top_k,
                                                         int vocab, int chunks, int list_max,
                                                         float* out, u32x2* __restrict__ list) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[4 * (kT1 / 64)];
  __shared__ uint32_t sel[2];
  const int row = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int t = threadIdx.x;
  const int len = min(kChunk, vocab - c * kChunk);
  const int keff = kept_count(top_k[row], vocab);
  if (!has_list(keff, len, list_max)) return;  // the second stage reads this chunk itself
  const float* src = probs + (size_t)row * vocab + (size_t)c * kChunk;
  float* dst = out + (size_t)row * vocab + (size_t)c * kChunk;

  // entry (j, e) of thread t is chunk entry 2048 j + 4 t + e
  uint32_t key[kRounds][4];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int l = 4 * (kT1 * j + t);
    if constexpr (kVec) {
      const f32x4 v = (l < len) ? *(const f32x4*)(src + l) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = rank_key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = (l + e < len) ? rank_key(src[l + e]) : 0u;
    }
  }
  auto valid = [&](int j, int e) { return 4 * (kT1 * j + t) + e < len; };

  // ---- radix select of the keff-th largest key of the chunk ----
  uint32_t prefix = 0, rem = (uint32_t)keff, count_eq = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = digit_shift(pass), nb = digit_bins(pass);
    const int prev_shift = pass == 1 ? 21 : 10;
    for (int i = t; i < kHistBins; i += kT1) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = key[j][e];
        if (valid(j, e) && (pass == 0 || (kk >> prev_shift) == prefix))
          atomicAdd(&hist[(kk >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    __syncthreads();
    find_digit<kT1>(hist, nb, rem, wsum, sel);
    const uint32_t d = sel[0];
    rem -= sel[1];
    prefix = pass == 0 ? d : ((prefix << (pass == 1 ? 11 : 10)) | d);
    if (pass == 2) count_eq = hist[d];
    __syncthreads();
  }
  const uint32_t T = prefix, need_eq = rem;  // keep keys > T and the first need_eq keys == T

  // ---- ranks of the ties (only when some of them are dropped) ----
  // Per round counts are packed two to a word (each round holds at most 2048 entries).
  bool cand[kRounds][4];
  uint32_t tie_base[kRounds];
  if (need_eq < count_eq) {
    u32x4 packed = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      uint32_t n = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) n += (valid(j, e) && key[j][e] == T) ? 1u : 0u;
      packed[j >> 1] += n << (16 * (j & 1));
    }
    u32x4 tot;
    const u32x4 incl = block_incl_scan4<kT1>(packed, wsum, &tot);
    uint32_t run = 0;  // ties in earlier rounds
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const uint32_t mine = (packed[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t upto = (incl[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      tie_base[j] = run + upto - mine;
      run += (tot[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRounds; ++j) tie_base[j] = 0;
  }
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    uint32_t r = tie_base[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kk = key[j][e];
      const bool tie = valid(j, e) && kk == T;
      cand[j][e] = valid(j, e) && (kk > T || (tie && r < need_eq));
      r += tie ? 1u : 0u;
    }
  }

  // ---- write the candidates in index order, zero the chunk's output ----
  u32x4 packed = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    uint32_t n = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) n += cand[j][e] ? 1u : 0u;
    packed[j >> 1] += n << (16 * (j & 1));
  }
  u32x4 tot;
  const u32x4 incl = block_incl_scan4<kT1>(packed, wsum, &tot);
  u32x2* lst = list + ((size_t)row * chunks + c) * list_max;
  uint32_t run = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const uint32_t mine = (packed[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t upto = (incl[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    uint32_t pos = run + upto - mine;
    run += (tot[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const int l = 4 * (kT1 * j + t);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (cand[j][e]) {
        lst[pos] = (u32x2){key[j][e], (uint32_t)(c * kChunk + l + e)};
        ++pos;
      }
    if constexpr (kVec) {
      if (l < len) *(f32x4*)(dst + l) = (f32x4){0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (l + e < len) dst[l + e] = 0.f;
    }
  }
}

template <bool kVec>
__global__ __launch_bounds__(kT2) void topk_row_kernel(const float* probs,
                                                       const int32_t* __restrict__ top_k,
                                                       int vocab, int chunks, int list_max,
                                                       float* out, const u32x2* __restrict__ list) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[kT2 / 64];
  __shared__ float fsum[kT2 / 64];
  __shared__ uint32_t sel[2];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int keff = kept_count(top_k[row], vocab);
  const float* src_row = probs + (size_t)row * vocab;
  float* dst_row = out + (size_t)row * vocab;

  // Every candidate of the row once, as (key, index): a chunk's list, or the chunk itself.
  auto for_each = [&](auto&& fn) {
    for (int c = 0; c < chunks; ++c) {
      const int len = min(kChunk, vocab - c * kChunk);
      if (has_list(keff, len, list_max)) {
        const u32x2* lst = list + ((size_t)row * chunks + c) * list_max;
        for (int j = t; j < keff; j += kT2) {
          const u32x2 e = lst[j];
          fn(e.x, e.y);
        }
      } else if constexpr (kVec) {
        const float* src = src_row + (size_t)c * kChunk;
#pragma unroll 4
        for (int j = 4 * t; j < len; j += 4 * kT2) {
          const f32x4 v = *(const f32x4*)(src + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) fn(rank_key(v[e]), (uint32_t)(c * kChunk + j + e));
        }
      } else {
        const float* src = src_row + (size_t)c * kChunk;
#pragma unroll 4
        for (int j = t; j < len; j += kT2) fn(rank_key(src[j]), (uint32_t)(c * kChunk + j));
      }
    }
  };
  long n = 0;  // candidates in all
  for (int c = 0; c < chunks; ++c) {
    const int len = min(kChunk, vocab - c * kChunk);
    n += has_list(keff, len, list_max) ? keff : len;
  }

  // Radix select of the rem-th largest of kf(key, idx) over the candidates that pass
  // `keep`; returns it, leaves in *rem how many entries equal to it are to be taken
  // and in *count_eq how many there are.
  auto select = [&](uint32_t rem0, auto&& keep, auto&& kf, uint32_t* rem, uint32_t* count_eq) {
    uint32_t prefix = 0, r = rem0;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = digit_shift(pass), nb = digit_bins(pass);
      const int prev_shift = pass == 1 ? 21 : 10;
      for (int i = t; i < kHistBins; i += kT2) hist[i] = 0;
      __syncthreads();
      for_each([&](uint32_t key, uint32_t idx) {
        if (!keep(key, idx)) return;
        const uint32_t kk = kf(key, idx);
        if (pass == 0 || (kk >> prev_shift) == prefix)
          atomicAdd(&hist[(kk >> shift) & (uint32_t)(nb - 1)], 1u);
      });
      __syncthreads();
      find_digit<kT2>(hist, nb, r, wsum, sel);
      const uint32_t d = sel[0];
      r -= sel[1];
      prefix = pass == 0 ? d : ((prefix << (pass == 1 ? 11 : 10)) | d);
      if (pass == 2) *count_eq = hist[d];
      __syncthreads();
    }
    *rem = r;
    return prefix;
  };

  // kept: key > T, or key == T and index <= cut
  uint32_t T = 0, cut = 0xFFFFFFFFu;
  bool all = n <= keff;
  if (!all) {
    uint32_t need_eq, count_eq;
    T = select((uint32_t)keff, [](uint32_t, uint32_t) { return true; },
               [](uint32_t key, uint32_t) { return key; }, &need_eq, &count_eq);
    if (need_eq < count_eq) {  // the need_eq tied entries of lowest index
      uint32_t r1, c1;
      const uint32_t T_ = T;
      cut = ~select(need_eq, [T_](uint32_t key, uint32_t) { return key == T_; },
                    [](uint32_t, uint32_t idx) { return ~idx; }, &r1, &c1);
    }
  }
  auto kept = [&](uint32_t key, uint32_t idx) {
    return all || key > T || (key == T && idx <= cut);
  };

  float s = 0.f;
  for_each([&](uint32_t key, uint32_t idx) {
    if (kept(key, idx)) s += key_value(key);
  });
  const float S = block_sum_f32<kT2>(s, fsum);

  for (int c = 0; c < chunks; ++c) {
    const int len = min(kChunk, vocab - c * kChunk);
    if (has_list(keff, len, list_max)) {
      // the first launch zeroed the chunk; only the kept candidates are written
      const u32x2* lst = list + ((size_t)row * chunks + c) * list_max;
      for (int j = t; j < keff; j += kT2) {
        const u32x2 e = lst[j];
        if (kept(e.x, e.y)) dst_row[e.y] = (S != 0.f) ? __fdiv_rn(key_value(e.x), S) : 0.f;
      }
    } else {
      const float* src = src_row + (size_t)c * kChunk;
      float* dst = dst_row + (size_t)c * kChunk;
      for (int j = t; j < len; j += kT2) {
        const float v = src[j];
        const bool k_ = kept(rank_key(v), (uint32_t)(c * kChunk + j));
        dst[j] = (k_ && S != 0.f) ? __fdiv_rn(v, S) : 0.f;
      }
    }
  }
}

}  // namespace

long top_k_chunks(int vocab) { return vocab > 0 ? (vocab + kChunk - 1) / kChunk : 0; }

hipError_t launch_top_k_renorm(const float* probs, const int32_t* top_k, int rows, int vocab,
                               int list_max, float* out, void* list, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const long chunks = top_k_chunks(vocab);
  const long g1 = rows * chunks;
  if (g1 > 0x7fffffffL) return hipErrorInvalidValue;
  const bool vec = (vocab % 4 == 0) && ((uintptr_t)probs % 16 == 0) && ((uintptr_t)out % 16 == 0);
  u32x2* l = (u32x2*)list;
  if (vec) {
    hipLaunchKernelGGL(topk_chunk_kernel<true>, dim3((unsigned)g1), dim3(kT1), 0, stream, probs,
                       top_k, vocab, (int)chunks, list_max, out, l);
    hipLaunchKernelGGL(topk_row_kernel<true>, dim3(rows), dim3(kT2), 0, stream, probs, top_k,
                       vocab, (int)chunks, list_max, out, (const u32x2*)l);
  } else {
    hipLaunchKernelGGL(topk_chunk_kernel<false>, dim3((unsigned)g1), dim3(kT1), 0, stream, probs,
                       top_k, vocab, (int)chunks, list_max, out, l);
    hipLaunchKernelGGL(topk_row_kernel<false>, dim3(rows), dim3(kT2), 0, stream, probs, top_k,
                       vocab, (int)chunks, list_max, out, (const u32x2*)l);
  }
  return hipGetLastError();
}

}  // namespace mla_impl
