// mla_decode.hip -- split-KV decode / speculative-verify kernel and LSE merge for gfx950.
//
// Work decomposition.  One work-group per (sequence b, key split s, 16-row
// block rb).  A sequence's R = P * H query rows share every latent row it
// reads (heads attend independently over one shared history, Kimi K3
// engineering report, section "并行度必须适配真正的形状"), so the grid is sized
// from key splits: long histories spread over many work-groups, which is what
// made the 12-head decode fast there, and short verify batches still fill the
// 256 CUs (same section: 48 work-groups were too few, 384 did better).
//
// Per work-group, four waves stream disjoint 16-token steps of the split.
// Each wave keeps its own online-softmax state and a 16-row x 512 fp32
// accumulator, so no wave waits for another until the split is done (the 16
// query rows sit in LDS, read by all four).  Per step:
//   1. every lane loads 8 (bf16) or 16 (fp8) key values of one token straight
//      from the paged cache into MFMA A-operand registers (16 B per load;
//      fp8 is widened to bf16 exactly); a ring of register buffers keeps the
//      next 2 (fp8) or 1 (bf16) steps in flight;
//   2. S^T[16 tokens x 16 rows] = K Q^T with 18 bf16 MFMA 16x16x32 (Q^T, the
//      B operand, is read from LDS three k-steps ahead of its MFMA);
//   3. masking and the online softmax run on the 4 scores each lane holds,
//      with cross-lane max / sum over the 4 lane groups of a row through the
//      VALU lane swaps (v_permlane16/32_swap, no LDS round trip); the running
//      max is only moved (and the accumulator rescaled) when it trails the
//      chunk max by more than 2^8, which keeps the rescale off the hot path;
//   4. the value part (first 512 dims) of the same registers goes to a per-wave
//      LDS tile, is read back transposed with ds_read_b64_tr_b16 and feeds
//      O^T[512 x 16] += V^T P^T with 32 bf16 MFMA 16x16x16; P stays in
//      registers because the score tile's layout is the B operand's layout.
// At the end the four waves merge through LDS and the work-group writes either
// the final rows (one split) or a partial (O_s / l_s, lse_s) for the merge.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla_impl {
using namespace mla_dev;

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 16;       // tokens per wave step
constexpr int kKSteps = 18;     // 576 / 32
constexpr int kVRow = 528;      // LDS row stride (bf16) of a wave's value tile (512 + 16 pad)
constexpr int kORow = 516;      // LDS row stride (fp32) of the merged output tile
constexpr float kSlack = 8.0f;  // log2 units a row's reference max may trail its true max

struct DecodeSmem {
  uint16_t q[16 * kDK];                 // 18,432 B: the row block's queries
  union {
    uint16_t v[kWaves][kStep * kVRow];  // 67,584 B: per-wave value tiles
    struct {
      float o[16 * kORow];              // merged 16 x 512 accumulator
      float m[kWaves][16];
      float l[kWaves][16];
      float row_m[16];
      float row_l[16];
    } red;
  };
};

// Dims held by lane group `grp` for k-step kk of the 576-wide contraction.
// bf16: 8 consecutive dims per k-step; fp8: one 16-byte load covers two
// k-steps.  The same map is used for keys and queries, so any permutation of
// the contraction index is fine.
template <bool kFp8>
__device__ __forceinline__ int kdim(int kk, int grp) {
  return kFp8 ? 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1) : 32 * kk + 8 * grp;
}

template <bool kFp8>
__global__ __launch_bounds__(256, 1) void decode_partial_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) DecodeSmem sm;
  constexpr int kLoads = kFp8 ? 9 : 18;  // 16-byte loads per lane per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // token (A rows) / query row (B, C columns)
  const int grp = lane >> 4;  // k-group (A, B) / 4-row group (C)

  // Work-group -> (sequence, split, row block).  The RB row blocks of one
  // (b, s) pair get ids congruent mod 8, so they land on one XCD and share its L2.
  const int per = 8 * p.RB;
  const int id = blockIdx.x;
  const int rb = (id % per) / 8;
  const int pair = (id / per) * 8 + (id % 8);
  if (pair >= p.pairs) return;
  const int b = pair / p.S;
  const int s = pair % p.S;

  const int L = p.seq_lens[b];
  const int lo = p.kv_begin ? max(p.kv_begin[b], 0) : 0;
  const int hi_all = p.kv_end ? min(p.kv_end[b], L) : L;
  const int base = lo & ~(kStep - 1);
  const int t_begin = base + s * p.chunk_tokens;
  const int t_end = (s == p.S - 1) ? hi_all : min(hi_all, t_begin + p.chunk_tokens);

  const int r = rb * 16 + col;
  const bool row_ok = r < p.R;
  const int hi_row = row_ok ? min(hi_all, L - p.P + r / p.H + 1) : lo;

  // The row block's queries go to LDS once (rows past R are zero); every step
  // reads its Q^T fragments (B operand of the score MFMA) from there, three
  // k-steps ahead of their MFMA, which keeps the 16 query rows out of the
  // register budget.
  for (int i = tid; i < 16 * (kDK / 8); i += 256) {
    const int row = i / (kDK / 8), c8 = i % (kDK / 8);
    const int rq = rb * 16 + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (rq < p.R) v = *(const u32x4*)(p.q + ((size_t)b * p.R + rq) * kDK + 8 * c8);
    *(u32x4*)(sm.q + row * kDK + 8 * c8) = v;
  }
  __syncthreads();
  const uint16_t* qsrc = sm.q + col * kDK;
  auto qfrag = [&](int kk) { return *(const bf16x8*)(qsrc + kdim<kFp8>(kk, grp)); };

  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;
  uint16_t* vt = sm.v[wave];
  const size_t row_bytes = kFp8 ? kDK : 2 * kDK;

  auto load_step = [&](int t0, u32x4* dst) {
    // all 16 tokens of an aligned step sit in one block; clamp into the visible
    // span so masked lanes read a real row of that block, never a poisoned slot
    const int blk = p.block_table[(size_t)b * p.max_blocks + t0 / p.block_size];
    const int t = min(max(t0 + col, lo), hi_all - 1);
    const uint8_t* krow = p.kv + ((size_t)blk * p.block_size + (t % p.block_size)) * row_bytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      dst[i] = *(const u32x4*)(krow + (kFp8 ? 64 * i + 16 * grp : 2 * (32 * i + 8 * grp)));
  };

  auto process_step = [&](const u32x4* raw, int t0) {
    // scores: lane (col, grp) gets tokens t0 + 4 * grp + i of query row `col`; the value
    // part of each fragment goes to this wave's LDS tile on the way (bf16, token-major).
    // Schedule: the Q^T fragments of three k-steps are read before the first MFMA,
    // then every MFMA is followed by the read of the fragment three steps later.
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    uint16_t* vrow = vt + col * kVRow;
    if constexpr (kFp8) {
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        bf16x8 ka, kb;
        fp8x16_to_bf16(raw[j], ka, kb);
        if (j < 8) {
          *(bf16x8*)(vrow + 64 * j + 16 * grp) = ka;
          *(bf16x8*)(vrow + 64 * j + 16 * grp + 8) = kb;
        }
        sc = mfma_16x16x32(ka, qfrag(2 * j), sc);
        sc = mfma_16x16x32(kb, qfrag(2 * j + 1), sc);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const bf16x8 k = __builtin_bit_cast(bf16x8, raw[kk]);
        if (kk < 16) *(bf16x8*)(vrow + 32 * kk + 8 * grp) = k;
        sc = mfma_16x16x32(k, qfrag(kk), sc);
      }
    }

    {
      constexpr int kDsRead = 0x100, kMfma = 0x8, kAhead = 3;
      __builtin_amdgcn_sched_group_barrier(kDsRead, kAhead, 0);
#pragma unroll
      for (int i = 0; i < kKSteps - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kMfma, kAhead, 0);
    }

    float sv[4];
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * grp + i;
      const bool vis = (t >= lo) && (t < hi_row);
      sv[i] = vis ? sc[i] * p.score_scale_log2 : -INFINITY;
      cm = fmaxf(cm, sv[i]);
    }
    cm = wave_max16x4(cm);
    const float mn = fmaxf(m_run, cm);
    const bool need = mn > m_run + kSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m_run - mn) : 1.f;
      if (need) m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    }
    const float mref = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = fast_exp2(sv[i] - mref);
      l_run += pv[i];
    }
    const bf16x4 pb = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
    const i16x4 pf = __builtin_bit_cast(i16x4, pb);

    wave_lds_fence();
    const uint16_t* vsrc = vt + (4 * grp + (col >> 2)) * kVRow + 4 * (col & 3);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      acc[m] = mfma_16x16x16(lds_read_tr16(vsrc + 16 * m), pf, acc[m]);
    }
    wave_lds_fence();
  };

  // A ring of kDepth register buffers per wave: the loads of the next kDepth - 1
  // steps are in flight while a step computes (one step moves 9 KB of fp8 or
  // 18 KB of bf16 rows per wave).  The loop is unrolled by kDepth so every buffer
  // index is a compile-time constant.
  constexpr int kDepth = kFp8 ? 3 : 2;
  constexpr int kStride = kStep * kWaves;
  const int t_first = t_begin + kStep * wave;
  const int n_steps = t_first < t_end ? (t_end - t_first + kStride - 1) / kStride : 0;
  // Every step issues the same loads (prefetches past the wave's last step re-read
  // that step), and the steady-state loop below has no branch around them, so the
  // compiler counts them exactly and keeps the whole ring in flight.
  u32x4 ring[kDepth][kLoads];
  const int last_t0 = t_first + (n_steps - 1) * kStride;
  if (n_steps > 0) {
#pragma unroll
    for (int u = 0; u < kDepth - 1; ++u) load_step(min(t_first + u * kStride, last_t0), ring[u]);
  }
  int i0 = 0;
  for (; i0 + kDepth <= n_steps; i0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int i = i0 + u;
      load_step(min(t_first + (i + kDepth - 1) * kStride, last_t0),
                ring[(u + kDepth - 1) % kDepth]);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before the step computes
      process_step(ring[u], t_first + i * kStride);
    }
  }
  // tail: fewer than kDepth steps remain and all of them are already loaded
#pragma unroll
  for (int u = 0; u < kDepth - 1; ++u)
    if (i0 + u < n_steps) process_step(ring[u], t_first + (i0 + u) * kStride);

  // ---- merge the four waves ----
  const float l_row = wave_sum16x4(l_run);
  __syncthreads();  // value tiles are dead from here on; the union is reused
  if (grp == 0) {
    sm.red.m[wave][col] = m_run;
    sm.red.l[wave][col] = l_row;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.red.m[w][col]);
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm.red.m[w][col];
    if (mw != -INFINITY) Lsum += sm.red.l[w][col] * fast_exp2(mw - M);
  }
  const float my_scale = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - M);
  if (wave == 0 && grp == 0) {
    sm.red.row_m[col] = M;
    sm.red.row_l[col] = Lsum;
  }
  // acc[m][i] = O[row col][dim 16 m + 4 grp + i]
  float* orow = sm.red.o + col * kORow + 4 * grp;
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        f32x4 v = acc[m] * my_scale;
        if (w > 0) v += *(const f32x4*)(orow + 16 * m);
        *(f32x4*)(orow + 16 * m) = v;
      }
    }
    __syncthreads();
  }

  const int orow_i = tid >> 4;  // 16 threads per output row
  const int rr = rb * 16 + orow_i;
  if (rr >= p.R) return;
  const float Mr = sm.red.row_m[orow_i];
  const float Lr = sm.red.row_l[orow_i];
  const float inv = (Lr > 0.f) ? p.out_scale / Lr : 0.f;
  const float lse_v = (Lr > 0.f) ? (Mr + fast_log2(Lr)) * kLn2 : -INFINITY;
  const size_t n = (size_t)b * p.R + rr;
  const float* src = sm.red.o + orow_i * kORow;
  if (p.S == 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = 4 * (tid & 15) + 64 * k;
      const f32x4 v = *(const f32x4*)(src + d) * inv;
      if (p.out_bf16) {
        const bf16x4 o = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
        *(bf16x4*)((uint16_t*)p.out + n * kDV + d) = o;
      } else {
        *(f32x4*)((float*)p.out + n * kDV + d) = v;
      }
    }
    if (p.lse && (tid & 15) == 0) p.lse[n] = lse_v;
  } else {
    const size_t pn = (size_t)s * p.B * p.R + n;
    if ((tid & 15) == 0) p.part_lse[pn] = lse_v;
    if (Lr > 0.f) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int d = 4 * (tid & 15) + 64 * k;
        *(f32x4*)(p.part_out + pn * kDV + d) = *(const f32x4*)(src + d) * inv;
      }
    }
  }
}

// One work-group of 128 threads per row; each thread owns 4 of the 512 dims.  The
// partial rows are loaded unconditionally (a split without keys for the row left
// its slot unwritten; its weight selects the value away), so the loads of several
// splits are in flight together.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_out,
                                                    const float* __restrict__ part_lse, int S,
                                                    int N, void* out, int out_bf16, float* lse) {
  const int n = blockIdx.x;
  const int d = 4 * threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_lse[(size_t)s * N + n]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      const float x = part_lse[(size_t)s * N + n];
      const float w = (x == -INFINITY) ? 0.f : expf(x - M);
      const f32x4 v = *(const f32x4*)(part_out + ((size_t)s * N + n) * kDV + d);
      L += w;
      if (w > 0.f) acc += w * v;
    }
    acc *= 1.f / L;
  }
  if (out_bf16) {
    const bf16x4 o = {(__bf16)acc.x, (__bf16)acc.y, (__bf16)acc.z, (__bf16)acc.w};
    *(bf16x4*)((uint16_t*)out + (size_t)n * kDV + d) = o;
  } else {
    *(f32x4*)((float*)out + (size_t)n * kDV + d) = acc;
  }
  if (lse && threadIdx.x == 0) lse[n] = (M == -INFINITY) ? -INFINITY : M + logf(L);
}

}  // namespace

int decode_grid_size(int pairs, int RB) { return ((pairs + 7) / 8) * 8 * RB; }

hipError_t launch_decode_partial(const DecodeParams& p, bool kv_fp8, hipStream_t stream) {
  const int grid = decode_grid_size(p.pairs, p.RB);
  if (grid == 0) return hipSuccess;
  if (kv_fp8)
    hipLaunchKernelGGL(decode_partial_kernel<true>, dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_partial_kernel<false>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_out, const float* part_lse, int S, int N, void* out,
                        int out_bf16, float* lse, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(N), dim3(128), 0, stream, part_out, part_lse, S, N, out,
                     out_bf16, lse);
  return hipGetLastError();
}

}  // namespace mla_impl
