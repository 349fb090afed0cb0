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
//  1. one 256-thread work-group per 8,192-entry chunk of a row holds the chunk
//     in registers (32 entries per thread) and finds the chunk's k-th largest
//     entry by a radix select on order-preserving 32-bit keys (digits of 11, 11
//     and 10 bits counted in an LDS histogram).  The chunk's k candidates (key,
//     index) go to the workspace in index order and its output range is
//     zero-filled; the row's top k are among the union of its chunks' top k.
//     For a row kept whole the work-group writes its chunk's sum instead.
//  2. one 1024-thread work-group per row: for a row kept whole it writes p / S
//     with S the sum of the chunk sums; otherwise it selects the row's k-th
//     largest among the candidates the same way (from LDS when they fit),
//     resolves ties at the threshold by a second select on the index, sums the
//     kept entries in a fixed order and writes p / sum at the kept positions.
// For k above the list limit (or a chunk not longer than k) a chunk keeps no
// list and the second launch reads its entries straight from the input; rows
// with such k are served by one work-group and run several times slower.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla_impl {
using namespace mla_dev;

namespace {

constexpr int kT1 = 256;                       // first-stage threads
constexpr int kRounds = 8;                     // float4 loads per first-stage thread
constexpr int kChunk = kRounds * 4 * kT1;      // 8,192 entries per chunk
constexpr int kPack = kRounds / 2;             // per-round counts packed two to a word
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
  v = wave_incl_scan(v);
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

// The same for W independent sums at once.  wsum holds W * NT / 64 words.
template <int NT, int W>
__device__ __forceinline__ void block_incl_scan_n(uint32_t (&v)[W], uint32_t* wsum,
                                                  uint32_t (&total)[W]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < W; ++q) v[q] = wave_incl_scan(v[q]);
  if (lane == 63)
#pragma unroll
    for (int q = 0; q < W; ++q) wsum[W * wv + q] = v[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < W; ++q) {
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const uint32_t w = wsum[W * i + q];
      before += (i < wv) ? w : 0u;
      tot += w;
    }
    v[q] += before;
    total[q] = tot;
  }
  __syncthreads();
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

// Radix select over the keys the threads feed through for_each(fn), for the rem
// largest of them.  Returns T with *rem_eq and *count_eq such that the selected
// keys are those > T plus rem_eq of the count_eq keys == T; when rem_eq ==
// count_eq that is every key >= T.  The passes stop early once every key left in
// the digit bin holding the rem-th largest is needed (then T is the bin's lowest
// key).  Every thread calls it; 1 <= rem <= the number of keys.
template <int NT, class ForEach>
__device__ __forceinline__ uint32_t block_select(uint32_t rem, ForEach&& for_each,
                                                 uint32_t* hist, uint32_t* wsum, uint32_t* sel,
                                                 uint32_t* rem_eq, uint32_t* count_eq) {
  uint32_t prefix = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = digit_shift(pass), nb = digit_bins(pass);
    const int prev_shift = pass == 1 ? 21 : 10;
    for (int i = threadIdx.x; i < kHistBins; i += NT) hist[i] = 0;
    __syncthreads();
    for_each([&](uint32_t kk) {
      if (pass == 0 || (kk >> prev_shift) == prefix)
        atomicAdd(&hist[(kk >> shift) & (uint32_t)(nb - 1)], 1u);
    });
    __syncthreads();
    find_digit<NT>(hist, nb, rem, wsum, sel);
    const uint32_t d = sel[0];
    rem -= sel[1];
    prefix = pass == 0 ? d : ((prefix << (pass == 1 ? 11 : 10)) | d);
    const uint32_t in_bin = hist[d];
    __syncthreads();
    if (pass == 2) {
      *count_eq = in_bin;
      break;
    }
    if (in_bin == rem) {  // the whole bin is taken: keys >= its lowest key
      *count_eq = 0;
      rem = 0;
      prefix <<= shift;
      break;
    }
  }
  *rem_eq = rem;
  return prefix;
}

// The row's kept count: k <= 0 or k >= vocab keeps all of it.
__device__ __forceinline__ int kept_count(int k, int vocab) {
  return (k <= 0 || k >= vocab) ? vocab : k;
}

// A chunk of len entries keeps a candidate list iff k < len and k <= list_max.
__device__ __forceinline__ bool has_list(int keff, int len, int list_max) {
  return keff < len && keff <= list_max;
}

__device__ __forceinline__ int chunk_len(int vocab, int c) { return min(kChunk, vocab - c * kChunk); }

template <bool kVec>
__global__ __launch_bounds__(kT1) void topk_chunk_kernel(const float* __restrict__ probs,
                                                         const int32_t* __restrict__ top_k,
                                                         int vocab, int chunks, int list_max,
                                                         float* out, u32x2* __restrict__ list,
                                                         float* __restrict__ sums) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[kPack * (kT1 / 64)];
  __shared__ float fsum[kT1 / 64];
  __shared__ uint32_t sel[2];
  const int row = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int t = threadIdx.x;
  const int len = chunk_len(vocab, c);
  const float* src = probs + (size_t)row * vocab + (size_t)c * kChunk;
  float* dst = out + (size_t)row * vocab + (size_t)c * kChunk;
  const int k_row = top_k[row];

  // entry (j, e) of thread t is chunk entry 4 (kT1 j + t) + e; the loads go out
  // before k is tested (a chunk the second stage reads itself wastes them).  The input
  // is read once and the zero fill written once, both with the nontemporal hint (whole
  // lines per wave-wide access: 49.2 -> 47.7 us on 128 rows x 163,840; the hint on the
  // loads alone was slower, 50.5).
  // Entries past the chunk's end get key 0, the lowest key: with k below the
  // chunk's length they can never be selected (they also lose every tie, having
  // the highest indices), so the selection needs no validity test.
  uint32_t key[kRounds][4];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int l = 4 * (kT1 * j + t);
    if constexpr (kVec) {
      const f32x4 v = (l < len) ? __builtin_nontemporal_load((const f32x4*)(src + l))
                                : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = (l < len) ? rank_key(v[e]) : 0u;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = (l + e < len) ? rank_key(src[l + e]) : 0u;
    }
  }
  auto valid = [&](int j, int e) { return 4 * (kT1 * j + t) + e < len; };
  const int keff = kept_count(k_row, vocab);
  const bool keep_all = keff >= vocab;
  if (!keep_all && !has_list(keff, len, list_max)) return;  // the second stage reads it

  if (keep_all) {  // the whole row is kept: this chunk's share of the normaliser
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += valid(j, e) ? key_value(key[j][e]) : 0.f;
    const float S = block_sum_f32<kT1>(s, fsum);
    if (t == 0) sums[(size_t)row * chunks + c] = S;
    return;
  }

  // ---- the chunk's keff-th largest key T ----
  uint32_t need_eq, count_eq;  // keys > T, and need_eq of the count_eq keys == T
  const uint32_t T = block_select<kT1>(
      (uint32_t)keff,
      [&](auto&& fn) {
#pragma unroll
        for (int j = 0; j < kRounds; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            fn(key[j][e]);
      },
      hist, wsum, sel, &need_eq, &count_eq);

  // ---- the ties: when some are dropped, the need_eq of lowest index stay ----
  uint32_t cut = 0xFFFFFFFFu;  // keep keys > T, and keys == T at local index <= cut
  if (need_eq != count_eq) {
    uint32_t r1, c1;  // local indices are unique: every selected ~index is >= the result
    cut = ~block_select<kT1>(
        need_eq,
        [&](auto&& fn) {
#pragma unroll
          for (int j = 0; j < kRounds; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (key[j][e] == T) fn(~(uint32_t)(4 * (kT1 * j + t) + e));
        },
        hist, wsum, sel, &r1, &c1);
  }
  // this thread's candidates as one bit per entry (bit 4 j + e): two registers
  uint64_t cm = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kk = key[j][e];
      if (kk > T || (kk == T && (uint32_t)(4 * (kT1 * j + t) + e) <= cut))
        cm |= (uint64_t)1 << (4 * j + e);
    }

  // ---- write the candidates in index order, zero the chunk's output ----
  uint32_t packed[kPack] = {}, incl[kPack], tot[kPack];
#pragma unroll
  for (int j = 0; j < kRounds; ++j)
    packed[j >> 1] += (uint32_t)__builtin_popcount((uint32_t)(cm >> (4 * j)) & 15u) << (16 * (j & 1));
#pragma unroll
  for (int q = 0; q < kPack; ++q) incl[q] = packed[q];
  block_incl_scan_n<kT1, kPack>(incl, wsum, tot);
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
      if (((cm >> (4 * j + e)) & 1) && l + e < len) {  // (candidates lie inside the chunk)
        lst[pos] = (u32x2){key[j][e], (uint32_t)(c * kChunk + l + e)};
        ++pos;
      }
    if constexpr (kVec) {
      if (l < len) __builtin_nontemporal_store((f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4*)(dst + l));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (l + e < len) dst[l + e] = 0.f;
    }
  }
}

constexpr int kStage = 4096;  // candidates the second stage keeps in LDS

template <bool kVec>
__global__ __launch_bounds__(kT2) void topk_row_kernel(const float* probs,
                                                       const int32_t* __restrict__ top_k,
                                                       int vocab, int chunks, int list_max,
                                                       float* out, const u32x2* __restrict__ list,
                                                       const float* __restrict__ sums) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[kT2 / 64];
  __shared__ float fsum[kT2 / 64];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t st_key[kStage];
  __shared__ uint32_t st_idx[kStage];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int keff = kept_count(top_k[row], vocab);
  const float* src_row = probs + (size_t)row * vocab;
  float* dst_row = out + (size_t)row * vocab;

  if (keff >= vocab) {
    // Whole row kept: p / S with S the sum of the first stage's chunk sums, in
    // chunk order.
    float S = 0.f;
    for (int i = 0; i < chunks; ++i) S += sums[(size_t)row * chunks + i];
    if constexpr (kVec) {
#pragma unroll 4
      for (int j = 4 * t; j < vocab; j += 4 * kT2) {
        const f32x4 v = *(const f32x4*)(src_row + j);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (S != 0.f) ? __fdiv_rn(v[e], S) : 0.f;
        *(f32x4*)(dst_row + j) = o;
      }
    } else {
#pragma unroll 4
      for (int j = t; j < vocab; j += kT2) dst_row[j] = (S != 0.f) ? __fdiv_rn(src_row[j], S) : 0.f;
    }
    return;
  }

  // Every candidate of the row once, in index order, as (key, index): a chunk's list,
  // or the chunk itself.
  auto for_each_global = [&](auto&& fn) {
    for (int c = 0; c < chunks; ++c) {
      const int len = chunk_len(vocab, c);
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
    const int len = chunk_len(vocab, c);
    n += has_list(keff, len, list_max) ? keff : len;
  }
  // Few candidates (small k) are read into LDS once; the passes below then cost no
  // global round trips.
  const bool staged = n <= kStage;
  if (staged) {
    // entry q of the candidate sequence: chunk c at offset o_c, position q - o_c; the
    // kStage / kT2 loads of a thread are issued together, then written to LDS
    uint32_t sk[kStage / kT2], si[kStage / kT2];
#pragma unroll
    for (int u = 0; u < kStage / kT2; ++u) {
      const int q = t + u * kT2;
      sk[u] = 0;
      si[u] = 0;
      if (q >= n) continue;
      int c = 0, o = 0;
      for (;; ++c) {
        const int len = chunk_len(vocab, c);
        const int nc = has_list(keff, len, list_max) ? keff : len;
        if (q < o + nc) break;
        o += nc;
      }
      const int len = chunk_len(vocab, c);
      if (has_list(keff, len, list_max)) {
        const u32x2 e = list[((size_t)row * chunks + c) * list_max + (q - o)];
        sk[u] = e.x;
        si[u] = e.y;
      } else {
        si[u] = (uint32_t)(c * kChunk + (q - o));
        sk[u] = rank_key(src_row[si[u]]);
      }
    }
#pragma unroll
    for (int u = 0; u < kStage / kT2; ++u) {
      const int q = t + u * kT2;
      if (q < n) {
        st_key[q] = sk[u];
        st_idx[q] = si[u];
      }
    }
    __syncthreads();
  }
  auto for_each = [&](auto&& fn) {
    if (staged) {
      for (int i = t; i < (int)n; i += kT2) fn(st_key[i], st_idx[i]);
    } else {
      for_each_global(fn);
    }
  };

  // kept: key > T, or key == T and index <= cut
  uint32_t T = 0, cut = 0xFFFFFFFFu;
  const bool all = n <= keff;
  if (!all) {
    uint32_t need_eq, count_eq;
    T = block_select<kT2>(
        (uint32_t)keff, [&](auto&& fn) { for_each([&](uint32_t key, uint32_t) { fn(key); }); },
        hist, wsum, sel, &need_eq, &count_eq);
    if (need_eq != count_eq) {  // the need_eq tied entries of lowest index
      uint32_t r1, c1;  // indices are unique: every selected ~index is >= the result
      cut = ~block_select<kT2>(
          need_eq,
          [&](auto&& fn) {
            for_each([&](uint32_t key, uint32_t idx) {
              if (key == T) fn(~idx);
            });
          },
          hist, wsum, sel, &r1, &c1);
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
  auto scaled = [&](float v) { return (S != 0.f) ? __fdiv_rn(v, S) : 0.f; };

  if (staged) {
    // a listed chunk was zeroed by the first stage: only its kept entries are written
    for (int i = t; i < (int)n; i += kT2) {
      const uint32_t key = st_key[i], idx = st_idx[i];
      const bool listed = has_list(keff, chunk_len(vocab, (int)(idx / kChunk)), list_max);
      if (kept(key, idx))
        dst_row[idx] = scaled(key_value(key));
      else if (!listed)
        dst_row[idx] = 0.f;
    }
    return;
  }
  for (int c = 0; c < chunks; ++c) {
    const int len = chunk_len(vocab, c);
    if (has_list(keff, len, list_max)) {
      const u32x2* lst = list + ((size_t)row * chunks + c) * list_max;
      for (int j = t; j < keff; j += kT2) {
        const u32x2 e = lst[j];
        if (kept(e.x, e.y)) dst_row[e.y] = scaled(key_value(e.x));
      }
    } else {
      const float* src = src_row + (size_t)c * kChunk;
      float* dst = dst_row + (size_t)c * kChunk;
      for (int j = t; j < len; j += kT2) {
        const float v = src[j];
        dst[j] = kept(rank_key(v), (uint32_t)(c * kChunk + j)) ? scaled(v) : 0.f;
      }
    }
  }
}

}  // namespace

long top_k_chunks(int vocab) { return vocab > 0 ? (vocab + kChunk - 1) / kChunk : 0; }

hipError_t launch_top_k_renorm(const float* probs, const int32_t* top_k, int rows, int vocab,
                               int list_max, float* out, void* list, float* sums,
                               hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const long chunks = top_k_chunks(vocab);
  const long grid = rows * chunks;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  const bool vec = (vocab % 4 == 0) && ((uintptr_t)probs % 16 == 0) && ((uintptr_t)out % 16 == 0);
  u32x2* l = (u32x2*)list;
  if (vec) {
    hipLaunchKernelGGL(topk_chunk_kernel<true>, dim3((unsigned)grid), dim3(kT1), 0, stream, probs,
                       top_k, vocab, (int)chunks, list_max, out, l, sums);
    hipLaunchKernelGGL(topk_row_kernel<true>, dim3(rows), dim3(kT2), 0, stream, probs,
                       top_k, vocab, (int)chunks, list_max, out, (const u32x2*)l,
                       (const float*)sums);
  } else {
    hipLaunchKernelGGL(topk_chunk_kernel<false>, dim3((unsigned)grid), dim3(kT1), 0, stream,
                       probs, top_k, vocab, (int)chunks, list_max, out, l, sums);
    hipLaunchKernelGGL(topk_row_kernel<false>, dim3(rows), dim3(kT2), 0, stream, probs,
                       top_k, vocab, (int)chunks, list_max, out, (const u32x2*)l,
                       (const float*)sums);
  }
  return hipGetLastError();
}

}  // namespace mla_impl
