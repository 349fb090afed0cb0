// mla_decode.hip -- persistent decode / speculative-verify kernel and LSE merge for gfx950.
//
// Work decomposition.  A sequence's R = P * H query rows share every latent row
// it reads (heads attend independently over one shared history, Kimi K3
// engineering report, section "并行度必须适配真正的形状"), so the unit of work is
// a 16-token step of one sequence for one 16-row block.  The steps of all
// sequences are laid end to end (each sequence also charged a few virtual steps
// for what a work-group pays per sequence it touches) and cut into W equal
// pieces; one work-group runs per (piece, row block), about one per CU, so a
// batch of uneven histories keeps every CU streaming until the end (the same
// section: the grid must be shaped to the real problem, 48 work-groups were too
// few, 384 did better).  A sequence spread over several pieces is merged in the
// same launch: each piece publishes (O / l, lse) for its share with
// agent-coherent stores and bumps a per-sequence counter; the piece that
// finishes last combines the shares by lse (the combination position-sharded
// attention uses, same report, section "缓存可复用，还要能一致地恢复") and resets
// the counter for the next call.  When a sequence is spread over many pieces
// (few sequences in the batch) that one merging CU would be the bottleneck, so
// the pieces only publish their shares and a second launch merges every output
// row in parallel.
//
// Per work-group, four waves stream interleaved 16-token steps of a segment.
// Each wave keeps its own online-softmax state and a 16-row x 512 fp32
// accumulator, so no wave waits for another until the segment is done; each
// wave holds the row block's 18 Q^T fragments in registers.  Per step:
//   1. the step's 16 latent rows come in with 16-byte loads per lane, a ring of
//      two register buffers keeping the next step in flight (block ids come
//      through the scalar cache a step early).  BF16: each lane loads its
//      MFMA A-operand fragments (8 key values of one token) straight from the
//      cache.  FP8: the step's 9 KB are loaded as whole 1 KB spans with the
//      nontemporal hint and written as they stand to a per-wave LDS stage, from
//      which the lanes read their fragments back (16 codes of one token,
//      widened to bf16 exactly);
//   2. S^T[16 tokens x 16 rows] = K Q^T with 18 bf16 MFMA 16x16x32 (Q^T, the
//      B operand, from registers);
//   3. masking and the softmax numerator run on the 4 scores each lane holds,
//      with cross-lane max / sum over the 4 lane groups of a row through the
//      VALU lane swaps (v_permlane16/32_swap, no LDS round trip); each row's
//      reference maximum is fixed at its first visible score, so the
//      accumulator is never rescaled inside the loop (see the step loop);
//   4. O^T[512 x 16] += V^T P^T, with P in registers as the score tile left it
//      (its layout is the B operand's).  BF16: the value part (first 512 dims)
//      of the fragments goes to a per-wave LDS tile and is read back transposed
//      with ds_read_b64_tr_b16 for 32 MFMA 16x16x16; step i + 1's score half
//      runs before step i's value half (two value tiles per wave).  FP8: two
//      steps at a time, V^T read from the two stages with ds_read_b64_tr_b8 and
//      widened, 32 MFMA 16x16x32 over the pair's 32 tokens.
// At the end of a segment the four waves merge through LDS and the work-group
// writes either the final rows (the piece holds the whole sequence) or its share.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla_impl {
using namespace mla_dev;

#ifdef MLA_TIMELINE
// per work-group: start, step-list scan done, then for its last segment: streaming loop
// end, wave merge done, result written or share published (counter bumped), merge done
__device__ unsigned long long decode_stamps[kStampGroups * kStampSlots];
#endif

namespace {

constexpr int kWaves = 4;
constexpr int kKSteps = 18;     // 576 / 32
constexpr int kVRow = 528;      // LDS row stride (bf16) of a wave's value tile (512 + 16 pad)
constexpr int kORow = 516;      // LDS row stride (fp32) of the merged output tile
constexpr float kCap = 64.0f;   // log2 units a score may exceed its row's reference max
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x2, kSchedMfma = 0x8, kSchedDsRead = 0x100;
// fp8 caches: a wave stages each step's 16 rows of codes in LDS, two steps at a time
constexpr int kSRow = kDK + 16;          // stage row stride in bytes (592)
constexpr int kStageB = kStep * kSRow + 128;  // second stage of a pair (9,600 B in)
constexpr int kPairBytes = 19200;        // a wave's pair of stages

struct DecodeSmem {
  union {
    uint16_t v[kWaves][2 * kStep * kVRow];  // 135,168 B: two value tiles per wave (bf16)
    uint8_t st[kWaves][kPairBytes];         //  76,800 B: a pair of step stages per wave (fp8)
    struct {
      float o[kWaves][16 * kORow];          // 132,096 B: each wave's scaled accumulator
      float m[kWaves][16];
      float l[kWaves][16];
      float lb[kWaves][16];
    } red;
  };
};

// The value tile of a wave is token-major with the 16-byte chunks of rows
// 8..15 swapped pairwise (chunk c stored at c ^ 1): a fragment write (16 rows,
// one chunk) then covers all 64 banks, and a transposed read (4 rows of one
// half) stays conflict-free.
template <bool kFp8>
__global__ __launch_bounds__(256, 1) void decode_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) DecodeSmem sm;
  __shared__ int last_flag;
  constexpr int kLoads = kFp8 ? 9 : 18;  // 16-byte loads per lane per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // token (A rows) / query row (B, C columns)
  const int grp = lane >> 4;  // k-group (A, B) / 4-row group (C)
  // Work-group -> (piece, row block).  In each complete group of 8 pieces the RB
  // row blocks of a piece get ids congruent mod 8, so they run on one XCD and read
  // the piece's rows through one L2; the last W % 8 pieces take the remaining ids
  // with their row blocks side by side, so the grid is exactly W x RB.
  const int W = p.W;
  const int per = 8 * p.RB;
  const int full = (W / 8) * per;
  const int id = blockIdx.x;
  MLA_STAMP(decode_stamps, 0);
  const int rb = id < full ? (id % per) / 8 : (id - full) % p.RB;
  const int w = id < full ? (id / per) * 8 + id % 8 : 8 * (W / 8) + (id - full) / p.RB;
  if (w >= W) return;
  const size_t row_bytes = kFp8 ? kDK : 2 * kDK;
  uint16_t* vt = sm.v[wave];

  // ---- the batch's step list: total N and where this piece starts ----
  // Each sequence with keys contributes p.seg_steps virtual steps followed by its
  // real 16-token steps; pieces are equal shares of that list.  The virtual steps
  // stand for what a piece pays per sequence it touches (query load, wave merge,
  // publishing a partial), so a piece that picks up a second sequence gets that
  // much less streaming.  256 sequences are read at a time, one per thread.
  // Piece 0 also writes the rows of sequences without visible keys: zeros and
  // lse = -inf.
  __shared__ long long red[kWaves];
  __shared__ long long seg[3];  // first sequence of the piece, its list offset, list length
  __shared__ int seg_range[4];  // L, lo, hi, n of that first sequence
  const int c = p.seg_steps;
  // the sequences without keys: piece 0 writes their rows (and, for the separate
  // merge, an empty share range)
  auto write_empty = [&](int b) {
    if (!p.merge_in_kernel && rb == 0) {
      p.seq_pieces[2 * b] = 0;  // no shares to merge
      p.seq_pieces[2 * b + 1] = 0;
    }
    for (int row = 0; row < 16; ++row) {
      const int rr = rb * 16 + row;
      if (rr >= p.R) break;
      const size_t n = io_row(p, b, rr);
      for (int d = 0; d < kDV; d += 4) store_row4(p, n, d, (f32x4){0.f, 0.f, 0.f, 0.f});
      if (p.lse) p.lse[n] = -INFINITY;
    }
  };
  long long N;
  if (p.B <= 64) {
    // One wave holds every sequence (one per lane): its sum, its scan and the search
    // for this piece's first sequence need no work-group barrier but the last.
    if (wave == 0) {
      const int b = lane;
      SeqRange sr = {0, 0, 0, 0, 0};
      if (b < p.B) sr = seq_range(p, b);
      const long long mb = sr.n > 0 ? sr.n + c : 0;
      if (w == 0 && b < p.B && sr.n == 0) write_empty(b);
      if (w == 0 && rb == 0 && b < p.B) check_lengths(p, b);
      long long incl, tot;
      if (!__builtin_amdgcn_ballot_w64(mb >= (1ll << 25))) {
        // every count below 2^25: the 32-bit register scan cannot overflow
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
      if (w == 0 && rb == 0) check_lengths(p, b);
    }
    if (tid == 0) seg[0] = p.B;
    N = block_sum(part, red);
  }
  // With fewer list entries than pieces only the first N pieces take part, so every
  // piece in use holds at least one entry: the pieces that share a sequence's real
  // steps are consecutive and each holds some of them.
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
      if (mb > 0 && ob <= S0 && S0 < ob + mb) {  // the one sequence holding entry S0
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
  long o = (long)seg[1];  // list offset of sequence b
  MLA_STAMP(decode_stamps, 1);

  for (int b = b_first; b < p.B && o < S1; ++b) {
    // the first sequence's range came with the scan; later ones are read here
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
    if (sr.n == 0) continue;  // empty sequences were written above
    const long rs = o + c;    // list offset of b's first real step
    o = rs + sr.n;
    const int a = (int)(max(S0, rs) - rs), e = (int)(min(S1, rs + sr.n) - rs);  // local steps
    if (e <= a) continue;  // only virtual entries of b fall in this piece
    const int lo = sr.lo, hi_all = sr.hi, L = sr.L;
    const int r = rb * 16 + col;
    const bool row_ok = r < p.R;
    const int hi_row = row_ok ? min(hi_all, L - p.P + r / p.H + 1) : lo;
    const int w_first = owner(rs, N, We), w_last = owner(rs + sr.n - 1, N, We);
    if (!p.merge_in_kernel && rb == 0 && w == w_first && tid == 0) {
      p.seq_pieces[2 * b] = w_first;  // the shares the separate merge combines
      p.seq_pieces[2 * b + 1] = w_last;
    }

    if (b != b_first) __syncthreads();  // the previous segment is done with the LDS tiles
    // The 18 Q^T fragments (B operand of the score MFMA) of the lane's query row stay
    // in registers for the whole segment, loaded straight from global memory before
    // the key prefetch: only MFMAs read them, so they can live in accumulation
    // registers, and no score MFMA waits on an LDS read.  Rows past R are zero.
    bf16x8 qreg[kKSteps];
    {
      const int rq = rb * 16 + col;
      const uint16_t* qrow = p.q + io_row(p, b, min(rq, p.R - 1)) * kDK;
  #pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const bf16x8 v = *(const bf16x8*)(qrow + kdim(kk, grp));
        qreg[kk] = rq < p.R ? v : (bf16x8){};
      }
    }
    auto qfrag = [&](int kk) { return qreg[kk]; };

    // Online softmax with a reference max that never moves inside the step loop.
    // A row's reference m_ref is its first visible score maximum (until then its
    // accumulator is zero, so setting it needs no rescale); later scores enter as
    // 2^(s - m_ref), which bf16 and fp32 hold exactly in range up to 2^kCap.  The
    // exponent is capped there, and m_max tracks the true maximum: a wave in which
    // some row went more than kCap above its reference runs its steps again, those
    // rows from their true maximum (no score can exceed it then), the others from
    // the same reference as before, so they come out bit-identical.  Keeping the
    // accumulator free of a data-dependent rescale keeps it in place in the
    // accumulation registers for the whole loop.
    f32x4 acc[32];
    float m_ref = -INFINITY;
    float m_max = -INFINITY;
    float l_run = 0.f;   // sum of the fp32 probabilities: the lse
    float lb_run = 0.f;  // sum of their bf16 roundings: the output's normaliser

    // Cache row of token t0 of an aligned step.  t0 is uniform, so the block id comes
    // through the scalar cache and stays out of the vector-load queue: a vector load
    // here would make every later wait on it drain the whole prefetch ring.
    const kconst_i32* bt = (const kconst_i32*)(p.block_table + (size_t)b * p.max_blocks);
    int ids_seen = 0;  // OR of the block ids read: negative if one was (flagged after the loop)
    auto step_row = [&](int t0) -> long {
      t0 = __builtin_amdgcn_readfirstlane(t0);
      const long id = kFp8 ? block_id(bt, t0 / p.block_size, ids_seen)
                           : block_id_now(p, bt, t0 / p.block_size);
      return id * p.block_size + t0 % p.block_size;
    };
    // Masking and the softmax numerator of one step's scores: lane (col, grp) holds
    // S^T[tokens t0 + 4 grp + i][query row col].  Returns the bf16 weights, which are
    // the value MFMA's B operand as they stand.
    auto weigh = [&](f32x4 sc, int t0) -> bf16x4 {
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
      m_max = fmaxf(m_max, cm);
      m_ref = (m_ref == -INFINITY) ? cm : m_ref;
      const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
      float pv[4];
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = fast_exp2(fminf(sv[i] - mref, kCap));
        l_run += pv[i];
      }
      // The value MFMA weighs the keys with P rounded to bf16; the output is
      // normalised by the sum of those same rounded weights (lb_run), so it is an
      // exact convex combination of the values it used and a key that dominates its
      // row contributes its value unchanged; lse keeps the exact fp32 sum l_run.
      const bf16x4 pb = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
  #pragma unroll
      for (int i = 0; i < 4; ++i) lb_run += (float)pb[i];
      return pb;
    };

    // BF16 caches.  Lanes load their MFMA fragments straight from the cache.
    auto load_step = [&](long row0, int t0, u32x4* dst) {
      // all 16 tokens of an aligned step sit in one block; clamping into the visible
      // span keeps every lane inside the step, on a real row, never a poisoned slot
      const int t = min(max(t0 + col, lo), hi_all - 1);
      const uint8_t* krow = p.kv + row0 * row_bytes + (t - t0) * (int)row_bytes;
  #pragma unroll
      for (int i = 0; i < kLoads; ++i) dst[i] = *(const u32x4*)(krow + 2 * kdim(i, grp));
    };

    // Score half of a step: the keys of step t0 (raw cache bytes) against the row
    // block's queries.  Lane (col, grp) gets tokens t0 + 4 grp + i of query row col;
    // the value part of each fragment goes to LDS tile `vt_w` on the way (bf16,
    // token-major).  Returns P^T as the B operand of the value MFMA.
    auto score_step = [&](const u32x4* raw, int t0, uint16_t* vt_w) -> i16x4 {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      // write bases: chunk 8 j + 2 grp + h of row col sits at chunk (8 j + 2 grp + (h ^ sw))
      const int sw = (col >> 3) & 1;
      uint16_t* vrow0 = vt_w + col * kVRow + 16 * grp + 8 * sw;        // h = 0
      uint16_t* vrow1 = vt_w + col * kVRow + 16 * grp + 8 * (sw ^ 1);  // h = 1
  #pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const bf16x8 k = __builtin_bit_cast(bf16x8, raw[kk]);
        if (kk < 16) *(bf16x8*)(((kk & 1) ? vrow1 : vrow0) + 64 * (kk >> 1)) = k;
        sc = mfma_16x16x32(k, qfrag(kk), sc);
      }
      return __builtin_bit_cast(i16x4, weigh(sc, t0));
    };

    // Value half of a step: O^T += V^T P^T from LDS tile `vt_r`, read transposed.
    // Lane (col, grp) addresses token 4 grp + col / 4, dims 16 m + 4 (col % 4) .. + 3.
    const int vr = 4 * grp + (col >> 2);
    const int v_lane = vr * kVRow + 8 * (((col & 3) >> 1) ^ ((vr >> 3) & 1)) + 4 * (col & 1);
    auto pv_step = [&](const uint16_t* vt_r, i16x4 pf) {
      const uint16_t* vsrc = vt_r + v_lane;
      // The transposed reads run kAheadV MFMAs ahead, so the LDS latency is paid
      // about once per step rather than once per MFMA.
      constexpr int kAheadV = 8;
      i16x4 vf[32];
  #pragma unroll
      for (int m = 0; m < 32; ++m) vf[m] = lds_read_tr16(vsrc + 16 * m);
  #pragma unroll
      for (int m = 0; m < 32; ++m) acc[m] = mfma_16x16x16(vf[m], pf, acc[m]);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kAheadV, 0);
  #pragma unroll
      for (int m = 0; m < 32 - kAheadV; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAheadV, 0);
    };

    // FP8 caches.  A step's 16 rows are 9,216 contiguous bytes, which every lane
    // loads as 16-byte pieces of whole 1 KB spans with the nontemporal hint (each
    // wave-wide load a run of full 128-byte lines: measured 6.2 - 6.5 TB/s, against
    // 5.7 - 5.8 for the fragment layout's 64-byte halves of lines, which the hint
    // only slows), and writes as they stand to a stage of 16 padded rows in LDS.
    // The score fragments are read back from the stage in the MFMA layout, and the
    // value operand with transposed 8-bit reads, widened to bf16 after the read;
    // only visible rows are read (row indices clamped into the span, as above), so
    // whatever the rows past a sequence's end hold never reaches the arithmetic.
    // Rows are 592 bytes apart and a pair's second stage starts 128 bytes (mod 256)
    // after the first: the 16 fragment reads of a 16-lane phase fall in 16 distinct
    // 16-byte bank groups, and each 32-lane half of a transposed read (16 rows, 8 from
    // each stage) in distinct banks.
    uint8_t* const stA = sm.st[wave];
    uint8_t* const stB = stA + kStageB;
    // A prefetch past the wave's last step (live false) still issues its loads, so the
    // waits stay exact, but every lane reads the same 16 bytes: one small request per
    // load instead of a re-read of the last step.
    auto load_codes = [&](long row0, u32x4* dst, bool live) {
      const u32x4* src = (const u32x4*)(p.kv + row0 * kDK) + (live ? lane : 0);
  #pragma unroll
      for (int i = 0; i < 9; ++i) dst[i] = __builtin_nontemporal_load(src + 64 * i);
    };
    // Score half: stage the codes of step t0, read back the lane's key fragments
    // (token t0 + col, dims 64 j + 16 grp .. + 15), widen and score them.
    auto stage_score = [&](const u32x4* raw, int t0, uint8_t* stage) -> bf16x4 {
  #pragma unroll
      for (int i = 0; i < 9; ++i) {
        const int u = 64 * i + lane;  // 16-byte piece u of the step: token u / 36
        *(u32x4*)(stage + (u / 36) * kSRow + 16 * (u % 36)) = raw[i];
      }
      wave_lds_fence();
      const int tk = min(max(t0 + col, lo), hi_all - 1) - t0;
      const uint8_t* kb = stage + tk * kSRow + 16 * grp;
      u32x4 kw[9];
  #pragma unroll
      for (int j = 0; j < 9; ++j) kw[j] = *(const u32x4*)(kb + 64 * j);
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int j = 0; j < 9; ++j) {
        bf16x8 ka, kb2;
        fp8x16_to_bf16(kw[j], ka, kb2);
        sc = mfma_16x16x32(ka, qfrag(2 * j), sc);
        sc = mfma_16x16x32(kb2, qfrag(2 * j + 1), sc);
      }
      // all nine reads first (left alone, the compiler waits for each read right
      // before its MFMAs: nine LDS round trips per step), then each fragment's
      // widening and its two MFMAs
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 9, 0);
  #pragma unroll
      for (int j = 0; j < 9; ++j) {
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      }
      return weigh(sc, t0);
    };
    // Value half of a pair of steps (t0a in stage A, t0b in stage B): O^T += V^T P^T
    // over their 32 tokens with 32 MFMA 16x16x32.  The MFMA's contraction index
    // 8 grp + e stands for token t0a + 4 grp + e (e < 4) or t0b + 4 grp + e - 4
    // (e >= 4), which is where the two steps' scores sit in P.  A transposed read gives
    // lane (col, grp) dim 16 m + col of the 8 tokens whose half-rows lanes 2 e and
    // 2 e + 1 of its group address.  Without a second step (pb = 0) the B half reads
    // stage A's rows again, finite values under zero weights.
    const int ve = col >> 1;
    auto stage_value = [&](int t0a, int t0b, bool has_b, bf16x4 pa, bf16x4 pb) {
      const bool in_b = has_b && ve >= 4;
      const int t0x = in_b ? t0b : t0a;
      const int tv = min(max(t0x + 4 * grp + (ve & 3), lo), hi_all - 1) - t0x;
      const uint8_t* vsrc = (in_b ? stB : stA) + tv * kSRow + 8 * (col & 1);
      const bf16x8 pf = __builtin_shufflevector(pa, pb, 0, 1, 2, 3, 4, 5, 6, 7);
      // The transposed reads run kAhead MFMAs ahead of their use, in a register ring
      // whose order a scheduling barrier per MFMA pins (left alone, the compiler
      // issues each read right before its widening and waits for it).
      constexpr int kAhead = 8;
      u32x2 vf[kAhead];
  #pragma unroll
      for (int m = 0; m < kAhead; ++m) vf[m] = lds_read_tr8(vsrc + 16 * m);
  #pragma unroll
      for (int m = 0; m < 32; ++m) {
        const bf16x8 v = fp8x8_to_bf16(vf[m % kAhead]);
        if (m + kAhead < 32) vf[m % kAhead] = lds_read_tr8(vsrc + 16 * (m + kAhead));
        acc[m] = mfma_16x16x32(v, pf, acc[m]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // A ring of two register buffers keeps the next step's loads in flight while a
    // step computes (one step moves 9 KB of fp8 or 18 KB of bf16 rows per wave).
    // BF16: the halves are software-pipelined: while the value MFMAs of step i run,
    // the same wave stores and scores step i + 1 (two LDS value tiles per wave
    // alternate).  FP8: steps go in pairs, each staged and scored in turn, then the
    // pair's values.
    constexpr int kDepth = 2;
    constexpr int kStride = kStep * kWaves;
    const int t_first = sr.base + kStep * (a + wave);
    const int n_steps = a + wave < e ? (e - a - wave + kWaves - 1) / kWaves : 0;
    // Every iteration issues the same loads (a prefetch past the wave's last step
    // re-reads that step, or for FP8 one 16-byte piece of it), so the compiler counts
    // them exactly and keeps the ring in flight.
    u32x4 ring[kDepth][kLoads];
    const int last_t0 = t_first + (n_steps - 1) * kStride;
    auto step_t0 = [&](int i) { return min(t_first + i * kStride, last_t0); };
    auto tile = [&](int i) { return vt + (i & 1) * (kStep * kVRow); };
    for (int pass = 0; pass < 2; ++pass) {
  #pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    lb_run = 0.f;
    if (n_steps > 0) {
      long row_next;  // cache row of the step the next prefetch loads (read a step early)
      if constexpr (kFp8) {
        load_codes(step_row(step_t0(0)), ring[0], true);
        load_codes(step_row(step_t0(1)), ring[1], n_steps > 1);
        row_next = step_row(step_t0(2));
        for (int i = 0; i < n_steps; i += 2) {
          const int ta = t_first + i * kStride, tb = ta + kStride;
          const bool has_b = i + 1 < n_steps;
          const bf16x4 pa = stage_score(ring[0], ta, stA);
          load_codes(row_next, ring[0], i + 2 < n_steps);  // step i + 2
          row_next = step_row(step_t0(i + 3));
          __builtin_amdgcn_sched_barrier(0);
          bf16x4 pb = {};
          if (has_b) pb = stage_score(ring[1], tb, stB);
          load_codes(row_next, ring[1], i + 3 < n_steps);  // step i + 3
          row_next = step_row(step_t0(i + 4));
          __builtin_amdgcn_sched_barrier(0);
          stage_value(ta, tb, has_b, pa, pb);
          wave_lds_fence();
        }
      } else {
  #pragma unroll
        for (int u = 0; u < kDepth; ++u) load_step(step_row(step_t0(u)), step_t0(u), ring[u]);
        row_next = step_row(step_t0(kDepth));
        i16x4 pf = score_step(ring[0], t_first, tile(0));
        wave_lds_fence();
        // iteration i: prefetch step i + kDepth into the slot step i left, score step
        // i + 1, accumulate step i
        auto body = [&](int i, const u32x4* raw_next, u32x4* slot_free) {
          load_step(row_next, step_t0(i + kDepth), slot_free);
          row_next = step_row(step_t0(i + kDepth + 1));
          __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before the step computes
          const i16x4 pf_next = score_step(raw_next, t_first + (i + 1) * kStride, tile(i + 1));
          pv_step(tile(i), pf);
          pf = pf_next;
          wave_lds_fence();
        };
        int i0 = 0;
        for (; i0 + kDepth < n_steps; i0 += kDepth) {
  #pragma unroll
          for (int u = 0; u < kDepth; ++u) body(i0 + u, ring[(u + 1) % kDepth], ring[u]);
        }
  #pragma unroll
        for (int u = 0; u < kDepth - 1; ++u)
          if (i0 + u + 1 < n_steps) body(i0 + u, ring[(u + 1) % kDepth], ring[u]);
        pv_step(tile(n_steps - 1), pf);
        wave_lds_fence();
      }
    }
    // a row beyond its cap: run the steps again from its true maximum
    if (!__builtin_amdgcn_ballot_w64(m_max > m_ref + kCap)) break;
    // only the rows that went past their cap move; the others recompute bit-identically
    m_ref = (m_max > m_ref + kCap) ? m_max : m_ref;
    }
    if (kFp8 && ids_seen < 0 && lane == 0) raise_flag(p, kFlagBadBlocks);

    MLA_STAMP(decode_stamps, 2);
    // ---- merge the four waves: one round through LDS ----
    const float l_row = wave_sum16x4(l_run);
    const float lb_row = wave_sum16x4(lb_run);
    __syncthreads();  // value tiles are dead from here on; the union is reused
    if (grp == 0) {
      sm.red.m[wave][col] = m_ref;
      sm.red.l[wave][col] = l_row;
      sm.red.lb[wave][col] = lb_row;
    }
    __syncthreads();
    {
      float M = -INFINITY;
  #pragma unroll
      for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm.red.m[v][col]);
      const float my_scale = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - M);
      // acc[m][i] = O[row col][dim 16 m + 4 grp + i]
      float* orow = sm.red.o[wave] + col * kORow + 4 * grp;
  #pragma unroll
      for (int m = 0; m < 32; ++m) *(f32x4*)(orow + 16 * m) = acc[m] * my_scale;
    }
    __syncthreads();

    MLA_STAMP(decode_stamps, 3);
    // ---- this piece's result for sequence b: final rows, or a partial + merge ----
    const int orow_i = tid >> 4;  // 16 threads per output row
    const int rr = rb * 16 + orow_i;
    const bool rr_ok = rr < p.R;
    float Mr = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) Mr = fmaxf(Mr, sm.red.m[v][orow_i]);
    float Lr = 0.f, Lb = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = sm.red.m[v][orow_i];
      if (mv != -INFINITY) {
        const float sc = fast_exp2(mv - Mr);
        Lr += sm.red.l[v][orow_i] * sc;
        Lb += sm.red.lb[v][orow_i] * sc;
      }
    }
    const float inv = (Lb > 0.f) ? p.out_scale / Lb : 0.f;
    const float lse_v = (Lr > 0.f) ? (Mr + fast_log2(Lr)) * kLn2 : -INFINITY;
    const size_t n = io_row(p, b, rr);
    // the four waves' scaled rows summed: dims d .. d + 3 of output row orow_i
    auto merged = [&](int d) {
      f32x4 x = *(const f32x4*)(sm.red.o[0] + orow_i * kORow + d);
  #pragma unroll
      for (int v = 1; v < kWaves; ++v) x += *(const f32x4*)(sm.red.o[v] + orow_i * kORow + d);
      return x;
    };
    if (w_first == w_last) {  // this piece holds the whole sequence
      if (rr_ok) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int d = 4 * (tid & 15) + 64 * k;
          store_row4(p, n, d, merged(d) * inv);
        }
        if (p.lse && (tid & 15) == 0) p.lse[n] = lse_v;
      }
      MLA_STAMP(decode_stamps, 4);
      continue;
    }
    const size_t slot = (size_t)(w + b) * p.R;  // slot w + b is unique per (piece, sequence)
    if (rr_ok) {
      if ((tid & 15) == 0) store_agent(p.part_lse + slot + rr, lse_v);
      if (Lr > 0.f) {
        const auto rsrc = agent_rsrc(p.part_out + slot * kDV);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int d = 4 * (tid & 15) + 64 * k;
          store_agent16(rsrc, (uint32_t)(rr * kDV + d) * 4, merged(d) * inv);
        }
      }
    }
    if (!p.merge_in_kernel) {  // a separate launch merges the shares
      MLA_STAMP(decode_stamps, 4);
      continue;
    }
    // Publish the partial; the last piece to finish sequence b merges all of them.
    // Every thread waits for its agent-coherent stores to be acknowledged before
    // the barrier, so they are visible device-wide before the counter moves; the
    // merging piece reads them with agent-coherent loads.  No fence, hence no
    // writeback or invalidation of the XCD's L2.
    wait_vm_all();
    __syncthreads();
    if (tid == 0) {
      int* cnt = p.counters + b * p.RB + rb;
      const int done = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = done == w_last - w_first;
      if (done > w_last - w_first) raise_flag(p, kFlagStaleCounters);  // not zero on entry
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = last;
    }
    __syncthreads();
    MLA_STAMP(decode_stamps, 4);
    if (!last_flag) continue;
    if (rr_ok) merge_pieces(p, b, rr, n, w_first, w_last);
#ifdef MLA_TIMELINE
    __syncthreads();
    MLA_STAMP(decode_stamps, 5);
#endif
  }
}

// The merge of sequences split into many shares, as a launch of its own: kQ
// 256-thread work-groups per output row, each owning 512 / kQ of its dims.  8 groups of
// 32 threads take every 8th share, each thread 16 / kQ dims, the loads of 4 kQ shares
// in flight per group (the same registers whatever kQ), combined online against a
// running maximum; the groups' results meet in LDS.  kQ = 4 takes a row's shares in a
// quarter of the rounds, for sequences spread over many pieces (one long sequence);
// kQ = 1 launches a quarter of the work-groups, for many rows with few shares each.
// The decode launch that wrote the shares has completed, so plain loads see them (the
// nontemporal hint on them cost the 1,024-key decode 1 us, and gained nothing elsewhere).  A
// share that saw no key of the row has lse = -inf and an unwritten row, which its
// zero weight selects away.
template <int kQ>
__global__ __launch_bounds__(256) void merge_shares_kernel(const DecodeParams p) {
  constexpr int kDims = kDV / kQ;        // dims of the row this work-group owns
  constexpr int kVec = 4 / kQ;           // f32x4 per thread and share
  constexpr int kBatch = 4 * kQ;         // shares in flight per group
  __shared__ float red[8][kDims + 4];
  __shared__ float gm[8], gl[8];
  const int tid = threadIdx.x;
  const size_t bn = blockIdx.x / kQ;  // row rr of sequence b of this launch's rows
  const int d0 = (int)(blockIdx.x % kQ) * kDims;
  const int b = (int)(bn / p.R), rr = (int)(bn % p.R);
  const size_t n = io_row(p, b, rr);
  const int w_first = p.seq_pieces[2 * b], w_last = p.seq_pieces[2 * b + 1];
  if (w_first == w_last) return;  // one piece held the whole sequence and wrote it
  const size_t R = p.R;
  const float* lse_b = p.part_lse + (size_t)b * R + rr;  // share v at v * R
  const int g = tid >> 5, l = tid & 31;
  f32x4 o4[kVec] = {};
  float mx = -INFINITY, ls = 0.f;
  for (int v0 = w_first + g; v0 <= w_last; v0 += 8 * kBatch) {
    float l4[kBatch];
    f32x4 t[kBatch][kVec];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int v = v0 + 8 * u;
      l4[u] = -INFINITY;
#pragma unroll
      for (int k = 0; k < kVec; ++k) t[u][k] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (v <= w_last) {  // past the end: no load, weight 0
        l4[u] = lse_b[v * R];
        const f32x4* src =
            (const f32x4*)(p.part_out + ((size_t)(v + b) * R + rr) * kDV + d0 + 4 * kVec * l);
#pragma unroll
        for (int k = 0; k < kVec; ++k) t[u][k] = src[k];
      }
    }
    float m_new = mx;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m_new = fmaxf(m_new, l4[u]);
    if (m_new == -INFINITY) continue;
    const float r = (mx == -INFINITY) ? 0.f : expf(mx - m_new);
    ls *= r;
#pragma unroll
    for (int k = 0; k < kVec; ++k) o4[k] *= r;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wt = (l4[u] == -INFINITY) ? 0.f : expf(l4[u] - m_new);
      ls += wt;
      if (wt > 0.f)
#pragma unroll
        for (int k = 0; k < kVec; ++k) o4[k] += wt * t[u][k];
    }
    mx = m_new;
  }
#pragma unroll
  for (int k = 0; k < kVec; ++k) *(f32x4*)&red[g][4 * kVec * l + 4 * k] = o4[k];
  if (l == 0) {
    gm[g] = mx;
    gl[g] = ls;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) M = fmaxf(M, gm[i]);
  float sc[8], wsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sc[i] = (gm[i] == -INFINITY) ? 0.f : expf(gm[i] - M);
    wsum += gl[i] * sc[i];
  }
  const float il = (M != -INFINITY && wsum > 0.f) ? 1.f / wsum : 0.f;
  // thread tid writes dims d0 + kDims / 256 * tid ..
  constexpr int kPer = kDims / 256;  // 2 (kQ = 1) or 0 (kQ = 4: half the threads write one)
  if constexpr (kPer == 2) {
    float2 v2 = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v2.x += red[i][2 * tid] * sc[i];
      v2.y += red[i][2 * tid + 1] * sc[i];
    }
    v2.x *= il;
    v2.y *= il;
    if (p.out_bf16) {
      const bf16x2 ob = {(__bf16)v2.x, (__bf16)v2.y};
      *(bf16x2*)((uint16_t*)p.out + n * kDV + d0 + 2 * tid) = ob;
    } else {
      *(float2*)((float*)p.out + n * kDV + d0 + 2 * tid) = v2;
    }
  } else if (tid < kDims) {
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) x += red[i][tid] * sc[i];
    x *= il;
    if (p.out_bf16)
      ((__bf16*)p.out)[n * kDV + d0 + tid] = (__bf16)x;
    else
      ((float*)p.out)[n * kDV + d0 + tid] = x;
  }
  if (p.lse && d0 == 0 && tid == 0) p.lse[n] = (M == -INFINITY) ? -INFINITY : M + logf(wsum);
}

// One work-group of 128 threads per row; each thread owns 4 of the 512 dims.  The
// partials are taken eight at a time, each batch's lse values loaded together with its
// rows and combined online against a running maximum, so up to eight partials cost one
// round trip to memory.  A partial that saw no key of the row has lse = -inf and an
// unwritten row, which its zero weight selects away.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_out,
                                                    const float* __restrict__ part_lse, int S,
                                                    int N, void* out, int out_bf16, float* lse) {
  constexpr int kBatch = 8;
  const int n = blockIdx.x;
  const int d = 4 * threadIdx.x;
  float mx = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float lv[kBatch];
    f32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = min(s0 + u, S - 1);  // past the end: re-read the last, weight 0
      lv[u] = (s0 + u < S) ? part_lse[(size_t)s * N + n] : -INFINITY;
      v[u] = *(const f32x4*)(part_out + ((size_t)s * N + n) * kDV + d);
    }
    float m_new = mx;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m_new = fmaxf(m_new, lv[u]);
    if (m_new == -INFINITY) continue;  // nothing seen yet
    const float r = (mx == -INFINITY) ? 0.f : expf(mx - m_new);
    L *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = (lv[u] == -INFINITY) ? 0.f : expf(lv[u] - m_new);
      L += w;
      if (w > 0.f) acc += w * v[u];
    }
    mx = m_new;
  }
  if (mx != -INFINITY) acc *= 1.f / L;
  if (out_bf16) {
    const bf16x4 o = {(__bf16)acc.x, (__bf16)acc.y, (__bf16)acc.z, (__bf16)acc.w};
    *(bf16x4*)((uint16_t*)out + (size_t)n * kDV + d) = o;
  } else {
    *(f32x4*)((float*)out + (size_t)n * kDV + d) = acc;
  }
  if (lse && threadIdx.x == 0) lse[n] = (mx == -INFINITY) ? -INFINITY : mx + logf(L);
}

__global__ __launch_bounds__(256) void clear_i32_kernel(int* p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int decode_grid_size(int W, int RB) { return W * RB; }

#ifdef MLA_TIMELINE
// Copies the stamps of the launches since the last read to host memory, then zeroes them.
extern "C" int mla_timeline_read_decode(void* host, size_t bytes) {
  void* dev = nullptr;
  if (bytes > sizeof(decode_stamps) || hipDeviceSynchronize() != hipSuccess ||
      hipMemcpyFromSymbol(host, HIP_SYMBOL(decode_stamps), bytes) != hipSuccess ||
      hipGetSymbolAddress(&dev, HIP_SYMBOL(decode_stamps)) != hipSuccess ||
      hipMemset(dev, 0, sizeof(decode_stamps)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return -1;
  return 0;
}
#endif

hipError_t launch_clear_i32(int* p, long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const long groups = (n + 255) / 256;
  if (groups > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(clear_i32_kernel, dim3((unsigned)groups), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, bool kv_fp8, hipStream_t stream) {
  const int grid = decode_grid_size(p.W, p.RB);
  if (grid == 0) return hipSuccess;
  if (kv_fp8)
    hipLaunchKernelGGL(decode_kernel<true>, dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<false>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge_shares(const DecodeParams& p, hipStream_t stream) {
  const long rows = (long)p.B * p.R;
  if (rows == 0) return hipSuccess;
  // one round of loads per row covers 32 shares with whole-row work-groups: split the
  // rows into quarters when the sequences average more shares than that
  const bool quarters = p.W > 32L * p.B;
  const long groups = rows * (quarters ? 4 : 1);
  if (groups > 0x7fffffffL) return hipErrorInvalidValue;
  if (quarters)
    hipLaunchKernelGGL(merge_shares_kernel<4>, dim3((unsigned)groups), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_shares_kernel<1>, dim3((unsigned)groups), dim3(256), 0, stream, p);
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
