// mla_verify.hip -- split-KV decode for sequences with more than 16 query rows (speculative
// verify: P positions x H heads) for gfx950.  One work-group per piece serves every
// 16-row block of the sequence, so each latent row is read from memory once per piece.
//
// The step list and the pieces are those of the one-row-block decode kernel: every
// sequence's key range in 16-token steps, laid end to end, each sequence charged a few
// virtual steps, cut into W equal pieces, one work-group per piece (about one per CU).
// Heads attend independently over one shared history (Kimi K3 engineering report,
// section "并行度必须适配真正的形状"), so the R = P * H rows of a sequence share every
// latent row: the piece's rows are copied once, 32 tokens at a time, from the paged cache
// into an LDS ring (coalesced 16-byte copies straight into LDS for BF16 caches; FP8 tiles
// are widened exactly to BF16 on the way in), and every wave reads them from there.
//
// Dataflow per 32-token tile (RB = 2..4 row blocks of 16 rows):
//   scores   wave rb (rb < RB) owns row block rb: S^T[32 tokens x 16 rows] = K Q^T by two
//            interleaved chains of 18 MFMA 16x16x32 (K fragments from LDS, Q^T in
//            registers for the whole segment), masking, online softmax against a per-row
//            reference fixed at the row's first visible score maximum (a row that goes
//            more than 64 log2 units past it makes the work-group run its segment again
//            from the true maximum); its weights P go to a small LDS buffer.
//   values   wave w owns value dims [128 w, 128 w + 128) of every row block:
//            O^T[128 x 16 rows] += V^T P^T, one MFMA 16x16x32 per 16 dims and row block,
//            each V^T operand (two transposed LDS reads) serving all RB row blocks.
// The score phase of tile k + 1 runs in the same interval as the value phase of tile k,
// one work-group barrier per tile.  Every row's weights come from one wave over its keys
// in order, the same arithmetic whatever RB, so head padding and head repetition leave
// the real rows bit-identical at a fixed piece count.
// A sequence split over several pieces is merged by lse exactly as in the decode kernel:
// in the launch by the last piece to finish it, or by the separate merge launch.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla_impl {
using namespace mla_dev;

#ifdef MLA_TIMELINE
// per work-group: start, step-list scan done, then for its last segment: queries and
// tile 0 in, first barrier of the tile loop, tile loop end, row normalisers shared,
// result written or share published
__device__ unsigned long long verify_stamps[kStampGroups * kStampSlots];
#endif

namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;                        // tokens per LDS tile (two steps)
constexpr int kKSteps = 18;                      // 576 / 32
constexpr int kPRowChunks = 73;                  // 16-byte chunks per padded LDS row (72 + pad)
constexpr int kPRow = 8 * kPRowChunks;           // padded LDS row, bf16 elements
constexpr int kDmaBlocks = 37;                   // 1 KB copy blocks that cover a padded tile
constexpr int kDmaPerWave = 10;                  // copies per wave and tile (spares repeat)
constexpr int kSlotBytes = kDmaBlocks * 1024;    // 37,888 B per tile slot
constexpr int kRingBf16 = 4;                     // tiles k (values), k + 1 (scores), two copying
constexpr int kRingFp8 = 3;                      // tiles k, k + 1, and k + 2 being written
constexpr int kDvWave = 128;                     // value dims per wave
constexpr int kKAhead = 4;                       // score chain: K fragments read this far ahead
constexpr int kVAhead = 3;                       // value MFMAs: V^T operands read this far ahead
constexpr float kCap = 64.0f;

static_assert(kTile * kPRowChunks <= kDmaBlocks * 64, "copy blocks must cover a tile");
static_assert(kWaves * kDmaPerWave >= kDmaBlocks, "the waves' copies must cover every block");

// FP8 tiles through registers: 16 codes per 16-byte load, widened exactly to bf16 into
// the padded tile layout.  32 rows x 36 chunks = 1,152 chunks, 4.5 per thread.
struct Fp8Stage {
  static constexpr int kRowChunks = kDK / 16;  // 36
  static constexpr int kTotal = kTile * kRowChunks;
  static constexpr int kChunks = (kTotal + 255) / 256;
  u32x4 r[kChunks];
};

template <bool kFp8, int kRB>
__global__ __launch_bounds__(256, 1) void verify_kernel(const DecodeParams p) {
  constexpr int kRing = kFp8 ? kRingFp8 : kRingBf16;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kSlotBytes];
  // a tile's weights P, double-buffered: [buffer][row block][row][contraction order k]
  __shared__ __attribute__((aligned(16))) __bf16 pbuf[2][kRB][16][kTile];
  // per row of each row block: reference maximum, fp32 weight sum, bf16 weight sum
  __shared__ float rowstat[kRB][3][16];
  __shared__ int last_flag;
  __shared__ int rerun;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // token (A rows) / query row (B, C columns)
  const int grp = lane >> 4;  // k-group (A, B) / 4-row group (C)
  const int W = p.W;
  const int w = blockIdx.x;
  MLA_STAMP(verify_stamps, 0);
  if (w >= W) return;
  const size_t row_bytes = kFp8 ? kDK : 2 * kDK;

  // wave w computes the scores of row block w (if w < RB) and value dims dv0 .. dv0 + 127
  const int my_rb = wave;
  const bool scorer = my_rb < kRB;
  const int dv0 = kDvWave * wave;

  // ---- the batch's step list: total N and where this piece starts (as in the decode
  // kernel); piece 0 writes the rows of sequences without visible keys ----
  __shared__ long long red[kWaves];
  __shared__ long long seg[3];
  __shared__ int seg_range[4];
  const int c = p.seg_steps;
  auto write_empty = [&](int b) {
    if (!p.merge_in_kernel) {
      p.seq_pieces[2 * b] = 0;
      p.seq_pieces[2 * b + 1] = 0;
    }
    for (int rr = 0; rr < p.R; ++rr) {
      const size_t n = io_row(p, b, rr);
      for (int d = 0; d < kDV; d += 4) store_row4(p, n, d, (f32x4){0.f, 0.f, 0.f, 0.f});
      if (p.lse) p.lse[n] = -INFINITY;
    }
  };
  long long N;
  if (p.B <= 64) {
    if (wave == 0) {
      const int b = lane;
      SeqRange sr = {0, 0, 0, 0, 0};
      if (b < p.B) sr = seq_range(p, b);
      const long long mb = sr.n > 0 ? sr.n + c : 0;
      if (w == 0 && b < p.B && sr.n == 0) write_empty(b);
      if (w == 0 && b < p.B) check_lengths(p, b);
      long long incl, tot;
      if (!__builtin_amdgcn_ballot_w64(mb >= (1ll << 25))) {
        const uint32_t i32 = wave_incl_scan((uint32_t)mb);
        incl = i32;
        tot = __builtin_amdgcn_readlane(i32, 63);
      } else {
        incl = mb;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const long long t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        tot = __shfl(incl, 63, 64);
      }
      const int We0 = (int)min((long long)W, tot);
      const long S0_ = w < We0 ? first_step(w, tot, We0) : 0;
      if (lane == 0) seg[2] = tot;
      if (w < We0 && mb > 0 && incl - mb <= S0_ && S0_ < incl) {
        seg[0] = b;
        seg[1] = incl - mb;
        seg_range[0] = sr.L;
        seg_range[1] = sr.lo;
        seg_range[2] = sr.hi;
        seg_range[3] = sr.n;
      }
    }
    __syncthreads();
    N = seg[2];
  } else {
    long long part = 0;
    for (int b0 = 0; b0 < p.B; b0 += 256) {
      const int b = b0 + tid;
      if (b >= p.B) break;
      const int nb = seq_range(p, b).n;
      part += nb > 0 ? nb + c : 0;
      if (w == 0 && nb == 0) write_empty(b);
      if (w == 0) check_lengths(p, b);
    }
    if (tid == 0) seg[0] = p.B;
    N = block_sum(part, red);
  }
  const int We = (int)min((long long)W, N);
  if (w >= We) return;
  const long S0 = first_step(w, N, We), S1 = first_step(w + 1, N, We);
  if (p.B > 64) {
    long long carry = 0;
    for (int b0 = 0; b0 < p.B; b0 += 256) {
      const int b = b0 + tid;
      SeqRange sr = {0, 0, 0, 0, 0};
      if (b < p.B) sr = seq_range(p, b);
      const long long mb = sr.n > 0 ? sr.n + c : 0;
      long long tot;
      const long long ob = carry + block_exclusive_scan(mb, red, &tot);
      if (mb > 0 && ob <= S0 && S0 < ob + mb) {
        seg[0] = b;
        seg[1] = ob;
        seg_range[0] = sr.L;
        seg_range[1] = sr.lo;
        seg_range[2] = sr.hi;
        seg_range[3] = sr.n;
      }
      carry += tot;
      __syncthreads();
      if (seg[0] < p.B) break;
    }
  }
  const int b_first = (int)seg[0];
  long o = (long)seg[1];
  MLA_STAMP(verify_stamps, 1);

  for (int b = b_first; b < p.B && o < S1; ++b) {
    SeqRange sr;
    if (b == b_first) {
      sr.L = seg_range[0];
      sr.lo = seg_range[1];
      sr.hi = seg_range[2];
      sr.n = seg_range[3];
      sr.base = sr.lo & ~(kStep - 1);
    } else {
      sr = seq_range(p, b);
    }
    if (sr.n == 0) continue;
    const long rs = o + c;
    o = rs + sr.n;
    const int a = (int)(max(S0, rs) - rs), e = (int)(min(S1, rs + sr.n) - rs);
    if (e <= a) continue;
    const int lo = sr.lo, hi_all = sr.hi, L = sr.L;
    const int r = my_rb * 16 + col;
    const bool row_ok = scorer && r < p.R;
    const int hi_row = row_ok ? min(hi_all, L - p.P + r / p.H + 1) : lo;
    const int w_first = owner(rs, N, We), w_last = owner(rs + sr.n - 1, N, We);
    if (!p.merge_in_kernel && w == w_first && tid == 0) {
      p.seq_pieces[2 * b] = w_first;
      p.seq_pieces[2 * b + 1] = w_last;
    }
    if (b != b_first) __syncthreads();  // the previous segment is done with the LDS buffers

    bf16x8 qreg[kKSteps];
    auto load_q = [&]() {
      if (scorer) {
        const uint16_t* qrow = p.q + io_row(p, b, min(r, p.R - 1)) * kDK;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const bf16x8 v = *(const bf16x8*)(qrow + kdim(kk, grp));
          qreg[kk] = r < p.R ? v : (bf16x8){};
        }
      }
    };

    // Cache rows of the tile's two 16-token halves.  A half lies inside one block (steps
    // are 16-aligned and blocks hold a multiple of 16 tokens); its tokens are clamped
    // into [lo, hi_all) so that every copy reads a real row of the same half (the
    // masked tokens' scores are discarded).  A half wholly past the range reads the
    // range's last row.
    const kconst_i32* bt = (const kconst_i32*)(p.block_table + (size_t)b * p.max_blocks);
    int ids_seen = 0;  // OR of the block ids read: negative if one was (flagged after the loop)
    const int n_tiles = (e - a + 1) / 2;
    const int tend = sr.base + kStep * e;  // tokens from here on belong to the next piece
    auto tile_t0 = [&](int k) { return sr.base + kStep * (a + 2 * k); };
    struct Half {
      long row0;  // cache row of token hb
      int hb;     // first token the half's rows are counted from
    };
    auto half_rows = [&](int th) -> Half {
      th = __builtin_amdgcn_readfirstlane(th);
      const int hb = th < hi_all ? th : ((hi_all - 1) & ~(kStep - 1));
      Half h;
      h.hb = hb;
      h.row0 = block_id(bt, hb / p.block_size, ids_seen) * p.block_size + hb % p.block_size;
      return h;
    };
    // byte address of token t's 16-byte chunk pc, for a token of half h
    auto chunk_addr = [&](const Half& h, int t, int pc) -> const uint8_t* {
      const int tc = min(max(t, lo), hi_all - 1);
      return p.kv + (size_t)(h.row0 + (tc - h.hb)) * row_bytes + 16 * pc;
    };
    auto slot_of = [&](int k) { return (const uint16_t*)(ring + (k % kRing) * kSlotBytes); };

    // BF16: copy tile k into slot k % kRing, 37 1 KB blocks, each wave ten of them.
    auto issue_tile = [&](int k) {
      const int T0 = tile_t0(k);
      const Half h0 = half_rows(T0), h1 = half_rows(T0 + kStep);
      const uint32_t slot = lds_addr(ring) + (uint32_t)((k % kRing) * kSlotBytes);
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const int inst = min(wave + 4 * i, kDmaBlocks - 1);
        const int pos = 64 * inst + lane;
        int row = pos / kPRowChunks, pc = pos - row * kPRowChunks;
        if (row >= kTile) row = kTile - 1;
        if (pc == kPRowChunks - 1) pc = 0;
        const uint8_t* src = chunk_addr(row < kStep ? h0 : h1, T0 + row, pc);
        dma16_addr(src, slot + 1024 * inst);
      }
    };
    // FP8: load tile k's codes into registers; widen and store them into slot k % kRing.
    auto fp8_load = [&](int k, Fp8Stage& st) {
      const int T0 = tile_t0(k);
      const Half h0 = half_rows(T0), h1 = half_rows(T0 + kStep);
#pragma unroll
      for (int j = 0; j < Fp8Stage::kChunks; ++j) {
        const int cidx = tid + 256 * j;
        if (cidx < Fp8Stage::kTotal) {
          const int row = cidx / Fp8Stage::kRowChunks, cc = cidx % Fp8Stage::kRowChunks;
          st.r[j] = *(const u32x4*)chunk_addr(row < kStep ? h0 : h1, T0 + row, cc);
        }
      }
    };
    auto fp8_store = [&](int k, const Fp8Stage& st) {
      uint16_t* buf = (uint16_t*)slot_of(k);
#pragma unroll
      for (int j = 0; j < Fp8Stage::kChunks; ++j) {
        const int cidx = tid + 256 * j;
        if (cidx < Fp8Stage::kTotal) {
          const int row = cidx / Fp8Stage::kRowChunks, cc = cidx % Fp8Stage::kRowChunks;
          bf16x8 lo8, hi8;
          fp8x16_to_bf16(st.r[j], lo8, hi8);
          *(bf16x8*)(buf + row * kPRow + 16 * cc) = lo8;
          *(bf16x8*)(buf + row * kPRow + 16 * cc + 8) = hi8;
        }
      }
    };

    f32x4 acc[kRB][kDvWave / 16];  // O^T of dims dv0 + 16 mt .. for each row block
    float m_ref = -INFINITY, m_max = -INFINITY;
    float l_run = 0.f, lb_run = 0.f;

    // Score phase (row-block owners): tile k's weights into pbuf[k % 2].  The tile's
    // tokens t0 .. t0 + 31 (those at or past tend belong to the next piece).  The two
    // halves' chains are interleaved.  The value MFMA's contraction index k = 8 g + i
    // stands for token 4 g + i (i < 4) of the first half and 16 + 4 g + (i - 4) of the
    // second: exactly the tokens lane (col, g) holds in its score registers, so each
    // lane's eight weights are one 16-byte store, read back as the B operand.
    // LDS operands are read a fixed distance ahead into register rings, and a scheduling
    // barrier after each group pins that order (left alone, the scheduler issues each read
    // right before its MFMA and waits for it: one LDS round trip per MFMA).
    auto score_finish = [&](f32x4 s0, f32x4 s1, int k) {
      const int t0 = tile_t0(k);
      float sv[8];
      float cm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = t0 + 4 * grp + (i & 3) + 16 * (i >> 2);
        const bool vis = (t >= lo) && (t < hi_row) && (t < tend);
        sv[i] = vis ? (i < 4 ? s0[i] : s1[i - 4]) * p.score_scale_log2 : -INFINITY;
        cm = fmaxf(cm, sv[i]);
      }
      cm = wave_max16x4(cm);
      m_max = fmaxf(m_max, cm);
      m_ref = (m_ref == -INFINITY) ? cm : m_ref;
      const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = fast_exp2(fminf(sv[i] - mref, kCap));
        l_run += pv;
        pb[i] = (__bf16)pv;
        lb_run += (float)pb[i];
      }
      *(bf16x8*)&pbuf[k & 1][my_rb][col][8 * grp] = pb;
    };
    // Value phase pieces for tile k: its weights, the V^T operand pointers, and one
    // 16-dim group (one MFMA per row block) with the ring refilled kVAhead groups ahead.
    struct ValueOps {
      bf16x8 pr[kRB];
      const uint16_t* v0;
      const uint16_t* v1;
      i16x4 x0[kVAhead], x1[kVAhead];
    };
    auto value_begin = [&](int k, ValueOps& vo) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) vo.pr[rb] = *(const bf16x8*)&pbuf[k & 1][rb][col][8 * grp];
      vo.v0 = slot_of(k) + (4 * grp + (col >> 2)) * kPRow + dv0 + 4 * (col & 3);
      vo.v1 = vo.v0 + 16 * kPRow;
#pragma unroll
      for (int i = 0; i < kVAhead; ++i) {
        vo.x0[i] = lds_read_tr16(vo.v0 + 16 * i);
        vo.x1[i] = lds_read_tr16(vo.v1 + 16 * i);
      }
    };
    auto value_group = [&](int mt, ValueOps& vo) {
      const int sl = mt % kVAhead;
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vo.x0[sl], vo.x1[sl], 0,
                                                                            1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) acc[rb][mt] = mfma_16x16x32(va, vo.pr[rb], acc[rb][mt]);
      if (mt + kVAhead < kDvWave / 16) {
        vo.x0[sl] = lds_read_tr16(vo.v0 + 16 * (mt + kVAhead));
        vo.x1[sl] = lds_read_tr16(vo.v1 + 16 * (mt + kVAhead));
      }
    };
    // Value phase of tile k.
    auto value_tile = [&](int k) {
      ValueOps vo;
      value_begin(k, vo);
#pragma unroll
      for (int mt = 0; mt < kDvWave / 16; ++mt) {
        value_group(mt, vo);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Score chains of tile k (two interleaved 16-token halves).
    auto score_tile = [&](int k) {
      const uint16_t* tile = slot_of(k);
      const uint16_t* k0 = tile + col * kPRow;
      const uint16_t* k1 = tile + (16 + col) * kPRow;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      bf16x8 ka[kKAhead], kb[kKAhead];
#pragma unroll
      for (int i = 0; i < kKAhead; ++i) {
        ka[i] = *(const bf16x8*)(k0 + kdim(i, grp));
        kb[i] = *(const bf16x8*)(k1 + kdim(i, grp));
      }
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const int sl = kk % kKAhead;
        s0 = mfma_16x16x32(ka[sl], qreg[kk], s0);
        s1 = mfma_16x16x32(kb[sl], qreg[kk], s1);
        if (kk + kKAhead < kKSteps) {
          ka[sl] = *(const bf16x8*)(k0 + kdim(kk + kKAhead, grp));
          kb[sl] = *(const bf16x8*)(k1 + kdim(kk + kKAhead, grp));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      score_finish(s0, s1, k);
    };
    // The queries load together with tile 0's copies, and both complete here, before the
    // segment loop: the compiler does not see the copies (asm), and a wait it placed for
    // the queries inside the tile loop would be a full vmcnt(0) that drains the copy ring
    // on every tile.  The queries go first (most come from L2; their latency then
    // overlaps the copies' instead of following it: 4 x 4 x 12-head verify 50.1 ->
    // 49.1 us).
    load_q();
    if constexpr (!kFp8) issue_tile(0);
    wait_vmcnt<0>();
    MLA_STAMP(verify_stamps, 2);
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int mt = 0; mt < kDvWave / 16; ++mt) acc[rb][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      l_run = 0.f;
      lb_run = 0.f;
      if (pass > 0) __syncthreads();  // the first pass is done with the LDS buffers
      // Tiles k (values) and k + 1 (scores) are read while tile k + 2 (and k + 3) arrive.
      Fp8Stage st;  // fp8: tile k + 2's codes, loaded one iteration ahead of their store
      if constexpr (kFp8) {
        fp8_load(0, st);
        fp8_store(0, st);
        if (n_tiles > 1) {
          fp8_load(1, st);
          fp8_store(1, st);
        }
        if (n_tiles > 2) fp8_load(2, st);
      } else {
        if (pass > 0) issue_tile(0);  // the first pass copied tile 0 with the queries
        if (n_tiles > 1) issue_tile(1);
        if (n_tiles > 2) issue_tile(2);
        // tile 0 and the queries in; the copies of tiles 1 and 2 may still fly
        if (n_tiles > 2)
          wait_vmcnt<2 * kDmaPerWave>();
        else if (n_tiles > 1)
          wait_vmcnt<kDmaPerWave>();
        else
          wait_vmcnt<0>();
      }
      __syncthreads();
      if (pass == 0) MLA_STAMP(verify_stamps, 3);
      if (scorer) score_tile(0);
      for (int k = 0; k < n_tiles; ++k) {
        if constexpr (kFp8) {
          // tile k + 1 was stored last iteration; the barrier also frees slot
          // (k + 2) % 3 (tile k - 1) and pbuf[(k + 1) % 2]
          __syncthreads();
          if (k + 2 < n_tiles) {
            fp8_store(k + 2, st);
            if (k + 3 < n_tiles) fp8_load(k + 3, st);
          }
        } else {
          // this wave's copies of tile k + 1 done (tile k + 2's may still fly), then every
          // wave's; the barrier also frees slot (k + 3) % 4 (tile k - 1) and
          // pbuf[(k + 1) % 2]
          if (k + 2 < n_tiles)
            wait_vmcnt<kDmaPerWave>();
          else
            wait_vmcnt<0>();
          __syncthreads();
          if (k + 3 < n_tiles) issue_tile(k + 3);
        }
        if (scorer && k + 1 < n_tiles) score_tile(k + 1);
        value_tile(k);
      }
      MLA_STAMP(verify_stamps, 4);
      // a row beyond its cap: the work-group runs the segment again, those rows from
      // their true maximum (the others recompute bit-identically)
      if (tid == 0) rerun = 0;
      __syncthreads();
      if (__builtin_amdgcn_ballot_w64(m_max > m_ref + kCap) && lane == 0) rerun = 1;
      __syncthreads();
      if (!rerun) break;
      m_ref = (m_max > m_ref + kCap) ? m_max : m_ref;
    }
    if (ids_seen < 0 && tid == 0) raise_flag(p, kFlagBadBlocks);

    MLA_STAMP(verify_stamps, 5);
    // ---- normalisers: the owners publish each row's, every wave scales its dims ----
    if (scorer) {
      const float l_row = wave_sum16x4(l_run), lb_row = wave_sum16x4(lb_run);  // whole wave
      if (grp == 0) {
        rowstat[my_rb][0][col] = m_ref;
        rowstat[my_rb][1][col] = l_row;
        rowstat[my_rb][2][col] = lb_row;
      }
    }
    __syncthreads();
    // final rows (this piece holds the whole sequence) or this piece's share of them;
    // acc[rb][mt][i] = O[row 16 rb + col][dim dv0 + 16 mt + 4 grp + i]
    const bool whole = w_first == w_last;
    const size_t slot_rows = (size_t)(w + b) * p.R;  // slot w + b is unique per (piece, sequence)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int rr = rb * 16 + col;
      if (rr >= p.R) continue;
      const float m = rowstat[rb][0][col], l = rowstat[rb][1][col], lb = rowstat[rb][2][col];
      const float inv = (lb > 0.f) ? p.out_scale / lb : 0.f;
      const float lse_v = (l > 0.f) ? (m + fast_log2(l)) * kLn2 : -INFINITY;
      const size_t n = io_row(p, b, rr);
      if (whole) {
#pragma unroll
        for (int mt = 0; mt < kDvWave / 16; ++mt)
          store_row4(p, n, dv0 + 16 * mt + 4 * grp, acc[rb][mt] * inv);
        if (p.lse && wave == 0 && grp == 0) p.lse[n] = lse_v;
      } else if (p.merge_in_kernel) {  // read by another piece of this launch: device-coherent
        if (wave == 0 && grp == 0) store_agent(p.part_lse + slot_rows + rr, lse_v);
        if (l > 0.f) {
          const auto rsrc = agent_rsrc(p.part_out + slot_rows * kDV);
#pragma unroll
          for (int mt = 0; mt < kDvWave / 16; ++mt)
            store_agent16(rsrc, (uint32_t)(rr * kDV + dv0 + 16 * mt + 4 * grp) * 4,
                          acc[rb][mt] * inv);
        }
      } else {  // read once by the merge launch that follows: plain stores, nontemporal
        if (wave == 0 && grp == 0) p.part_lse[slot_rows + rr] = lse_v;
        if (l > 0.f) {
          float* dst = p.part_out + (slot_rows + rr) * kDV + dv0 + 4 * grp;
#pragma unroll
          for (int mt = 0; mt < kDvWave / 16; ++mt)
            __builtin_nontemporal_store(acc[rb][mt] * inv, (f32x4*)(dst + 16 * mt));
        }
      }
    }
    MLA_STAMP(verify_stamps, 6);
    if (whole) continue;
    if (!p.merge_in_kernel) continue;  // a separate launch merges the shares
    // publish, then the last piece of the sequence merges every share (as in the decode
    // kernel: stores acknowledged before the counter moves, agent-coherent loads)
    wait_vm_all();
    __syncthreads();
    if (tid == 0) {
      int* cnt = p.counters + (size_t)b * p.RB;
      const int done = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = done == w_last - w_first;
      if (done > w_last - w_first) raise_flag(p, kFlagStaleCounters);  // not zero on entry
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = last;
    }
    __syncthreads();
    if (!last_flag) continue;
    for (int rr = tid >> 4; rr < p.R; rr += 16)
      merge_pieces(p, b, rr, io_row(p, b, rr), w_first, w_last);
  }
}

}  // namespace

#ifdef MLA_TIMELINE
// Copies the stamps of the launches since the last read to host memory, then zeroes them.
extern "C" int mla_timeline_read_verify(void* host, size_t bytes) {
  void* dev = nullptr;
  if (bytes > sizeof(verify_stamps) || hipDeviceSynchronize() != hipSuccess ||
      hipMemcpyFromSymbol(host, HIP_SYMBOL(verify_stamps), bytes) != hipSuccess ||
      hipGetSymbolAddress(&dev, HIP_SYMBOL(verify_stamps)) != hipSuccess ||
      hipMemset(dev, 0, sizeof(verify_stamps)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return -1;
  return 0;
}
#endif

hipError_t launch_verify_shared(const DecodeParams& p, bool kv_fp8, hipStream_t stream) {
  if (p.W <= 0) return hipSuccess;
  const dim3 grid(p.W), block(256);
#define MLA_VERIFY_LAUNCH(FP8, RB) \
  hipLaunchKernelGGL((verify_kernel<FP8, RB>), grid, block, 0, stream, p)
  switch (p.RB) {
    case 2:
      if (kv_fp8) MLA_VERIFY_LAUNCH(true, 2); else MLA_VERIFY_LAUNCH(false, 2);
      break;
    case 3:
      if (kv_fp8) MLA_VERIFY_LAUNCH(true, 3); else MLA_VERIFY_LAUNCH(false, 3);
      break;
    case 4:
      if (kv_fp8) MLA_VERIFY_LAUNCH(true, 4); else MLA_VERIFY_LAUNCH(false, 4);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef MLA_VERIFY_LAUNCH
  return hipGetLastError();
}

}  // namespace mla_impl
