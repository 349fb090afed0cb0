// mla_prefill.hip -- causal MLA prefill (absorbed form) for gfx950.
//
// Every query row is a (token, head) pair; the heads of a token share the
// token's latent rows and its causal limit.  The slow 12-head case on the
// pages was one attention kernel that only had fast shapes for 4, 8 or
// multiples of 16 heads (article on Kimi K3 on MI355X, section
// "首Token等待优化：简单补零解决大问题"); here rows are simply (token, head)
// pairs, so any head count tiles the same way.
//
// Work decomposition.  A work-group owns 128 consecutive query rows of one
// sequence; each of its four waves owns 32 of them, with the waves' Q^T
// fragments held in registers for the whole key loop (36 x 8 bf16 per lane).
// The work-group walks the sequence's keys in 32-token tiles up to its last
// row's token; each tile is copied once into an LDS ring as the cache holds it
// (bf16, or fp8 codes: padded rows, 1 KB global->LDS copies, two tiles in flight)
// and read by all four waves:
//   S^T[32 tokens x 32 rows] = K Q^T           36 MFMA 32x32x16 (A from LDS; fp8
//                                               codes 16 per read, widened exactly
//                                               after the read)
//   causal mask, online softmax against a per-row reference fixed from the first
//   tile before the key loop
//   O^T[512 x 32 rows] += V^T P^T               32 MFMA 32x32x16 (A = V^T read
//                                               with ds_read_b64_tr_b16, or for fp8
//                                               with ds_read_b64_tr_b8 and widened;
//                                               B = P^T straight from the score
//                                               registers)
// Work-groups are launched longest-first (the last rows of a sequence see the
// most keys), and consecutive ids fan out over the 8 XCDs, so every XCD works
// on a mix of long and short rows that all stream the same leading key tiles.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla_impl {
using namespace mla_dev;

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowsPerWg = 128;
constexpr int kRowsPerWave = 32;
constexpr int kTile = 32;                        // key tokens per tile
constexpr int kKSteps = 36;                      // 576 / 16
constexpr int kRing = 4;                         // tiles: two in use, two in flight
constexpr float kCap = 64.0f;  // log2 units a score may exceed its row's reference max
constexpr int kKAhead = 3;     // K fragments read this many score MFMAs ahead
constexpr int kVAhead = 3;     // V^T operands read this many value MFMAs ahead

// LDS layout of a tile: 32 rows of the cache's codes as they stand (bf16, or fp8 for
// fp8 caches), each padded by one 16-byte chunk, filled by 1 KB global->LDS copies.
template <bool kFp8>
struct Layout {
  static constexpr int kRowBytes = kFp8 ? kDK : 2 * kDK;             // 576 / 1152
  static constexpr int kPRowChunks = kRowBytes / 16 + 1;             // 37 / 73: data + 1 pad
  static constexpr int kPRowBytes = 16 * kPRowChunks;                // 592 / 1168
  static constexpr int kDmaBlocks = (kTile * kPRowChunks + 63) / 64; // 19 / 37 1 KB blocks
  static constexpr int kDmaPerWave = (kDmaBlocks + 3) / 4;           // 5 / 10 (the last repeats)
  static constexpr int kSlotBytes = kDmaBlocks * 1024;
  static_assert(kTile * kPRowChunks <= kDmaBlocks * 64, "DMA slots must cover a tile");
  static_assert(4 * kDmaPerWave >= kDmaBlocks, "the waves' copies must cover every block");
};

// Copy key tile [tok0, tok0 + 32) of a sequence into an LDS slot laid out as
// 32 padded rows.  Chunk positions past the tile land in the slot's slack; pad chunks
// and rows past the sequence end get real (masked) rows.  seq_kv points at the
// sequence's first latent row.
template <bool kFp8>
__device__ __forceinline__ void dma_tile(const uint8_t* seq_kv, int len, int tok0, uint32_t slot,
                                         int wave, int lane) {
  using L = Layout<kFp8>;
  // keep the per-lane chunk coordinates out of loop-invariant code motion: ten
  // of them held across the key loop would cost 20 VGPRs
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int i = 0; i < L::kDmaPerWave; ++i) {
    // block wave + 4 i; the waves' spare copies repeat the last block (same bytes)
    const int inst = min(wave + 4 * i, L::kDmaBlocks - 1);
    const int pos = 64 * inst + l;
    int row = pos / L::kPRowChunks, pc = pos - row * L::kPRowChunks;
    if (row >= kTile) row = kTile - 1;
    if (pc == L::kPRowChunks - 1) pc = 0;
    const int t = min(tok0 + row, len - 1);
    dma16(seq_kv, (uint32_t)(t * L::kRowBytes + 16 * pc), slot + 1024 * inst);
  }
}

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool kFp8>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const PrefillParams p) {
  using L = Layout<kFp8>;
  constexpr int KA = kKAhead, VA = kVAhead;
  // a ring of 4 tile slots: 148 KB of bf16 rows, 76 KB of fp8 codes
  __shared__ __attribute__((aligned(16))) uint8_t lds[kRing * L::kSlotBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // query row within the wave (B / C column)
  const int g = lane >> 5;   // k-group (A, B) / row group of 4 (C)

  // ---- work-group -> (sequence, row block), longest first within a sequence
  int id = blockIdx.x;
  int b = 0, len = 0, seq_start = 0, blk = -1;
  for (; b < p.B; ++b) {
    seq_start = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq_start;
    const int nb = (len * p.H + kRowsPerWg - 1) / kRowsPerWg;
    if (id < nb) {
      blk = nb - 1 - id;
      break;
    }
    id -= nb;
  }
  if (blk < 0) return;
  const int rows = len * p.H;
  const int row0 = blk * kRowsPerWg;
  const int wg_last_tok = min(len - 1, (row0 + kRowsPerWg - 1) / p.H);
  const int wg_first_tok = row0 / p.H;
  const int n_tiles = wg_last_tok / kTile + 1;

  // ---- this lane's query row and its Q^T fragments (B operand, 8 dims per k-step).
  // k-step kk covers dims 16 kk .. + 15, lane group g eight of them; for fp8 tiles,
  // whose fragments come 16 codes per read, k-steps 2 j and 2 j + 1 cover dims
  // 32 j .. + 31 with lane group g holding 32 j + 16 g + 8 (kk % 2) .. + 7 (the same
  // permutation of the contraction index on both sides).
  const int r = row0 + kRowsPerWave * wave + n;
  const bool row_ok = r < rows;
  const int tq = row_ok ? r / p.H : -1;  // causal limit: keys 0 .. tq
  bf16x8 qf[kKSteps];
  {
    const uint16_t* qrow =
        p.q + ((size_t)seq_start * p.H + (row_ok ? r : 0)) * kDK + (kFp8 ? 16 : 8) * g;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      bf16x8 v = *(const bf16x8*)(qrow + (kFp8 ? 32 * (kk >> 1) + 8 * (kk & 1) : 16 * kk));
      qf[kk] = row_ok ? v : (bf16x8){};
    }
  }
  // retire the query loads here: a wait the compiler would otherwise place at
  // their first use inside the key loop would also drain the tile copies in flight
  wait_vmcnt<0>();

  // Online softmax with a reference max that never moves inside the key loop: a
  // row's reference is its maximum over the first tile (key 0, visible to every
  // row, is in it); every score enters as 2^(s - m_ref), exact in bf16 and fp32 up
  // to 2^kCap, while x_max tracks the largest s - m_ref.  If any row of the
  // work-group went more than kCap above its reference, that pass is discarded and
  // the whole work-group runs the key loop again from zeroed sums, those rows from
  // their true maxima and the others from unchanged references (bit-identical
  // results).  With no data-dependent rescale the accumulator stays in its registers
  // for the loop.
  f32x16 acc[16];
  float m_ref = -INFINITY;
  float x_max = -INFINITY;  // this lane's largest score relative to the reference
  bool first_pass = true;
  float l_run = 0.f;   // sum of the fp32 probabilities: the lse
  float lb_run = 0.f;  // sum of their bf16 roundings: the output's normaliser

  // per-lane LDS byte offsets inside a tile.  K fragment: token n, byte 16 g of each
  // 32-byte step (bf16: dims 16 kk + 8 g; fp8: the 16 codes of dims 32 j + 16 g).
  const int a_off = n * L::kPRowBytes + 16 * g;
  // V^T: bf16, lane (l & 15) of a 16-lane group addresses token 4 g + (l & 15) / 4,
  // dims 4 (l & 3) .. + 3 of the group's 16 (ds_read_b64_tr_b16, second read 8 tokens
  // on); fp8, it addresses half-row (l & 1) of token 8 (e / 4) + 4 g + e % 4,
  // e = (l & 15) / 2 (ds_read_b64_tr_b8: the group's 8 tokens and 16 dims)
  const int ve = (lane & 15) >> 1;
  int v_off = kFp8 ? (8 * (ve >> 2) + 4 * g + (ve & 3)) * L::kPRowBytes + 16 * ((lane >> 4) & 1) +
                         8 * (lane & 1)
                   : (4 * g + ((lane & 15) >> 2)) * L::kPRowBytes + 32 * ((lane >> 4) & 1) +
                         8 * (lane & 3);
  // one opaque per-lane offset: the loop adds the tile's slot to it once and every
  // transposed read takes its constant part in the instruction's offset field
  asm volatile("" : "+v"(v_off));

  // Rows whose token precedes the whole tile are fully masked (their P is 0);
  // they still run the MFMAs: an early exit here would split the accumulator's
  // live range and cost far more than the few skipped diagonal tiles.
  // S^T of one tile: K fragments KA MFMAs ahead in a register ring; the order is pinned
  // by scheduling barriers (left alone, the scheduler issues each read right before
  // its MFMA and waits for it, exposing the LDS latency once per MFMA)
  auto scores = [&](const uint8_t* buf) {
    f32x16 sc = {};
    if constexpr (kFp8) {
      // 16 codes per read, two k-steps each, widened exactly after the read
      u32x4 kr[KA + 1];
#pragma unroll
      for (int j = 0; j < KA; ++j) kr[j] = *(const u32x4*)(buf + a_off + 32 * j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kKSteps / 2; ++j) {
        bf16x8 lo, hi;
        fp8x16_to_bf16(kr[j % (KA + 1)], lo, hi);
        if (j + KA < kKSteps / 2) kr[(j + KA) % (KA + 1)] = *(const u32x4*)(buf + a_off + 32 * (j + KA));
        sc = mfma_32x32x16(lo, qf[2 * j], sc);
        sc = mfma_32x32x16(hi, qf[2 * j + 1], sc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      bf16x8 kb[KA + 1];
#pragma unroll
      for (int kk = 0; kk < KA; ++kk) kb[kk] = *(const bf16x8*)(buf + a_off + 32 * kk);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        sc = mfma_32x32x16(kb[kk % (KA + 1)], qf[kk], sc);
        if (kk + KA < kKSteps)
          kb[(kk + KA) % (KA + 1)] = *(const bf16x8*)(buf + a_off + 32 * (kk + KA));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return sc;
  };
  // Each row's reference: its maximum over tile 0 (key 0 is visible to every row), set
  // once before the key loop from a score chain of its own, so the loop carries no
  // first-tile code.  The row's other 16 tokens sit in lane l ^ 32.
  auto set_reference = [&](const uint8_t* buf) {
    const f32x16 sc = scores(buf);
    const int lim = tq - 4 * g;
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      cm = fmaxf(cm, (8 * (i >> 2) + (i & 3) <= lim) ? sc[i] * p.score_scale_log2 : -INFINITY);
    m_ref = wave_max_xor32(cm);
  };

  auto compute = [&](const uint8_t* buf, int kt) {
    {
      const f32x16 sc = scores(buf);
      // lane (n, g) holds tokens kt*32 + 8 (i/4) + 4 g + i%4 of row n.  Scores are
      // taken relative to the row's reference: x = s * scale - m_ref in one fma.
      const int lim = tq - kt * kTile - 4 * g;
      const bool whole = kt * kTile + kTile - 1 <= wg_first_tok;  // every key visible to every row
      const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
      float xv[16];
      if (whole) {
#pragma unroll
        for (int i = 0; i < 16; ++i) xv[i] = __builtin_fmaf(sc[i], p.score_scale_log2, -mref);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xv[i] = (8 * (i >> 2) + (i & 3) <= lim)
                      ? __builtin_fmaf(sc[i], p.score_scale_log2, -mref) : -INFINITY;
      }
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x_max = fmaxf(x_max, xv[i]);
        // no clamp: a pass in which some x exceeds kCap (where 2^x could overflow) is
        // discarded and run again from zeroed sums, so only x <= kCap reach the output
        pv[i] = fast_exp2(xv[i]);
        l_run += pv[i];
      }
      // k-slot 8 g + s of k-step j holds token 16 j + 8 (s / 4) + 4 g + s % 4: exactly
      // the score values i = 8 j + s this lane already has
      // the value MFMA weighs the keys with P rounded to bf16, and the output is
      // normalised by the sum of those same weights (an exact convex combination of
      // the values: a key that dominates its row contributes its value unchanged),
      // summed pairwise by a bf16 dot product with (1, 1)
      bf16x8 pf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const bf16x2 pair = {(__bf16)pv[8 * j + i], (__bf16)pv[8 * j + i + 1]};
          pf[j][i] = pair.x;
          pf[j][i + 1] = pair.y;
          lb_run = __builtin_amdgcn_fdot2_f32_bf16(pair, (bf16x2){(__bf16)1.0f, (__bf16)1.0f},
                                                   lb_run, false);
        }
      }
      // V^T operands VA MFMAs ahead in a register ring, pinned the same way; MFMA m
      // covers dims 32 (m / 2) .. + 31 and keys 16 (m % 2) .. + 15
      if constexpr (kFp8) {
        // the ring holds the raw codes; each operand is widened at its MFMA
        auto vread8 = [&](int m) {
          return lds_read_tr8(buf + v_off + 16 * (m & 1) * L::kPRowBytes + 32 * (m >> 1));
        };
        u32x2 vr[VA + 1];
#pragma unroll
        for (int m = 0; m < VA; ++m) vr[m] = vread8(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 32; ++m) {
          const bf16x8 v = fp8x8_to_bf16(vr[m % (VA + 1)]);
          if (m + VA < 32) vr[(m + VA) % (VA + 1)] = vread8(m + VA);
          acc[m >> 1] = mfma_32x32x16(v, pf[m & 1], acc[m >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        auto vread = [&](int m) {
          const uint8_t* src = buf + v_off + 16 * (m & 1) * L::kPRowBytes + 64 * (m >> 1);
          const i16x4 lo = lds_read_tr16(src);
          const i16x4 hi = lds_read_tr16(src + 8 * L::kPRowBytes);
          const i16x8 v8 = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          return __builtin_bit_cast(bf16x8, v8);
        };
        bf16x8 vb[VA + 1];
#pragma unroll
        for (int m = 0; m < VA; ++m) vb[m] = vread(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 32; ++m) {
          acc[m >> 1] = mfma_32x32x16(vb[m % (VA + 1)], pf[m & 1], acc[m >> 1]);
          if (m + VA < 32) vb[(m + VA) % (VA + 1)] = vread(m + VA);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = (f32x16){};
  l_run = 0.f;
  lb_run = 0.f;
  {
    // tile kt lives in slot kt % 4
    const uint32_t base = lds_addr(lds);
    const uint8_t* seq_kv = p.kv + (size_t)seq_start * L::kRowBytes;
    // Byte offsets of this lane's ten chunks within a tile, fixed for the whole loop: a
    // tile that lies inside the sequence takes them as they are, its first row folded
    // into the scalar base; only the sequence's last, partial tile clamps rows.
    uint32_t dma_off[L::kDmaPerWave];
#pragma unroll
    for (int i = 0; i < L::kDmaPerWave; ++i) {
      const int pos = 64 * min(wave + 4 * i, L::kDmaBlocks - 1) + lane;
      int row = pos / L::kPRowChunks, pc = pos - row * L::kPRowChunks;
      if (row >= kTile) row = kTile - 1;
      if (pc == L::kPRowChunks - 1) pc = 0;
      dma_off[i] = (uint32_t)(row * L::kRowBytes + 16 * pc);
    }
    auto copy_tile = [&](int tok0, uint32_t slot) {
      if (tok0 + kTile <= len) {
        const uint8_t* tile_kv = seq_kv + (size_t)tok0 * L::kRowBytes;
#pragma unroll
        for (int i = 0; i < L::kDmaPerWave; ++i)
          dma16(tile_kv, dma_off[i], slot + 1024 * min(wave + 4 * i, L::kDmaBlocks - 1));
      } else {
        dma_tile<kFp8>(seq_kv, len, tok0, slot, wave, lane);
      }
    };
    copy_tile(0, base);
    if (n_tiles > 1) copy_tile(kTile, base + L::kSlotBytes);
    if (first_pass) {
      if (n_tiles > 1)
        wait_vmcnt<L::kDmaPerWave>();  // this wave's copies of tile 0 have landed
      else
        wait_vmcnt<0>();
      __syncthreads();
      set_reference(lds);
    }
    // Tiles go in pairs: one wait and one work-group barrier per two tiles.  At an even
    // tile kt the copies in flight are tiles kt and kt + 1 (issued two tiles earlier);
    // once everyone's have landed, tiles kt - 2 and kt - 1 are no longer read and their
    // slots take tiles kt + 2 and kt + 3.
    for (int kt = 0; kt < n_tiles; ++kt) {
      if ((kt & 1) == 0) {
        wait_vmcnt<0>();
        __syncthreads();
        if (kt + 2 < n_tiles) copy_tile((kt + 2) * kTile, base + ((kt + 2) % kRing) * L::kSlotBytes);
        if (kt + 3 < n_tiles) copy_tile((kt + 3) * kTile, base + ((kt + 3) % kRing) * L::kSlotBytes);
      }
      compute(lds + (kt % kRing) * L::kSlotBytes, kt);
    }
  }
  // a row beyond its cap anywhere in the work-group: all waves run the loop again
  x_max = wave_max_xor32(x_max);  // the row's (its tokens sit in lanes l and l ^ 32)
  if (!__syncthreads_or(x_max > kCap)) break;
  // only the rows that went past their cap move, to their true maximum; the others
  // recompute bit-identically
  m_ref = (x_max > kCap) ? m_ref + x_max : m_ref;
  x_max = -INFINITY;
  first_pass = false;
  }

  // ---- finalize this lane's row
  const float l_row = wave_sum_xor32(l_run);
  const float lb_row = wave_sum_xor32(lb_run);
  if (!row_ok) return;
  const float inv = (lb_row > 0.f) ? p.out_scale / lb_row : 0.f;
  const size_t orow = (size_t)seq_start * p.H + r;
  if (p.lse && g == 0)
    p.lse[orow] = (l_row > 0.f) ? (m_ref + fast_log2(l_row)) * kLn2 : -INFINITY;
  // acc[mb][i]: dim 32 mb + 8 (i / 4) + 4 g + i % 4
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * mb + 8 * q4 + 4 * g;
      const f32x4 v = {acc[mb][4 * q4] * inv, acc[mb][4 * q4 + 1] * inv,
                       acc[mb][4 * q4 + 2] * inv, acc[mb][4 * q4 + 3] * inv};
      if (p.out_bf16) {
        const bf16x4 o = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
        *(bf16x4*)((uint16_t*)p.out + orow * kDV + d) = o;
      } else {
        *(f32x4*)((float*)p.out + orow * kDV + d) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, bool kv_fp8, hipStream_t stream) {
  // upper bound on row blocks over all sequences; surplus work-groups exit at once
  const long blocks = ((long)p.T * p.H + kRowsPerWg - 1) / kRowsPerWg + p.B;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (kv_fp8)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla_impl
