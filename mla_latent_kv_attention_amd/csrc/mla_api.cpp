// mla_api.cpp -- the C-ABI entry points declared in include/mla.h.
//
// Host work only: argument checks (before any launch), the piece planner of the
// persistent decode, the workspace carve-up and the kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "mla.h"
#include "mla_kernels.h"

namespace {

constexpr int kStepTokens = 16;        // tokens per step of the concatenated step list
constexpr int kMinStepsPerPiece = 2;   // a short batch still spreads over many CUs
constexpr int kMaxPiecesPerSeq = 16;   // mean shares per sequence the in-launch merge takes
// What a piece pays for each sequence it touches (query load, wave merge, partial
// publish), in 16-token steps of streaming; measured per cache dtype.
constexpr int kSegmentStepsFp8 = 30;
constexpr int kSegmentStepsBf16 = 18;
constexpr int kMaxPieces = 1 << 16;
constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

int g_cu_count[kMaxDevices];  // 0 = not yet queried

int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int R, RB, W;
  bool merge_in_kernel;  // few enough shares per sequence for the last piece to merge them
  bool shared;           // one work-group per piece for all row blocks (launch_verify_shared)
};

// Sequences of more than 16 query rows take the kernel whose work-group serves all of a
// piece's row blocks (each latent row read once per piece) when the batch's key range is
// long, where streaming dominates: 4 sequences x 4 positions x 32,768 keys, 12 heads:
// 54.6 us against 64.4 us with one work-group per row block, 16 heads 62.9 against 84.
// Shorter batches keep one work-group per (piece, row block): there the shares the
// pieces publish (one fp32 row per query row and piece) outweigh the keys once a piece
// serves all row blocks of a 256-piece plan (one 32,768-key FP8 sequence x 4 positions:
// 32.1 us against 23.8 us).
constexpr long kSharedMinTokens = 65536;  // batch x longest key range

bool use_shared(int B, int RB, int max_kv_len) {
  return RB >= 2 && (long)(B > 0 ? B : 1) * max_kv_len >= kSharedMinTokens;
}

// Piece plan.  The kernel is persistent: W pieces x RB row blocks work-groups,
// one per CU (a work-group's LDS keeps it alone on its CU), each streaming an
// equal share of the batch's 16-token steps.  Short batches get fewer pieces
// so that every piece keeps its four waves busy; the max_kv_len hint only sizes
// W, and a wrong hint costs time, never correctness.
Plan make_plan(int B, int P, int H, int max_kv_len, int num_splits, int cus) {
  Plan pl;
  pl.R = P * H;
  pl.RB = (pl.R + 15) / 16;
  pl.shared = use_shared(B, pl.RB, max_kv_len);
  const long Bn = B > 0 ? B : 1;
  if (num_splits > 0) {
    pl.W = num_splits < kMaxPieces ? num_splits : kMaxPieces;
    pl.merge_in_kernel = pl.W <= kMaxPiecesPerSeq * Bn;
    return pl;
  }
  // one work-group per CU, so no piece waits for a CU to free up: the grid is W x RB
  // work-groups with one per (piece, row block), W with one per piece (shared)
  long W = (cus > 0 ? cus : 256) / (pl.shared ? 1 : pl.RB);
  const long steps = Bn * (((long)max_kv_len + kStepTokens - 1) / kStepTokens);
  const long by_steps = (steps + kMinStepsPerPiece - 1) / kMinStepsPerPiece;
  if (W > by_steps) W = by_steps;
  // The piece that finishes a sequence last merges every share of it through one
  // CU, which stays cheap up to kMaxPiecesPerSeq shares per sequence.  Beyond that
  // a separate launch merges every row in parallel.  The piece count is never cut
  // to keep the merge in the launch: idle CUs cost more than the second launch
  // (measured: 8 sequences x 17,750 keys, 37 us at 128 pieces, 27 us at 256 with
  // the separate merge; 4 sequences x 4 positions x 32,768 keys, 83 us at 64
  // pieces, 67 us at 80).
  const long cap = kMaxPiecesPerSeq * Bn;
  if (W < 1) W = 1;
  pl.W = (int)W;
  pl.merge_in_kernel = pl.W <= cap;
  return pl;
}

// Workspace: a fixed block of completion counters at offset 0 and the error-flags word
// after it (their place and size do not depend on the call's shape, so a workspace that
// calls of any shape leave zero stays zero there), then the partial rows and lse of the
// (W + B) slots.  One piece needs none.
constexpr size_t kCounterBytes = (size_t)MLA_MAX_COUNTERS * sizeof(int) + kAlign;  // + flags
static_assert(MLA_WORKSPACE_FLAGS_OFFSET == MLA_MAX_COUNTERS * sizeof(int), "flags word");

size_t workspace_bytes_for(const Plan& pl, int B) {
  if (pl.W <= 1) return 0;
  const size_t rows = (size_t)(pl.W + B) * pl.R;
  return kCounterBytes + align_up(rows * MLA_HEAD_DIM_V * sizeof(float)) +
         align_up(rows * sizeof(float)) + align_up((size_t)2 * B * sizeof(int));
}

bool finite_positive(float x) { return std::isfinite(x) && x > 0.f; }

mla_status check_dtype_out(int out_dtype) {
  return (out_dtype == MLA_DTYPE_FP32 || out_dtype == MLA_DTYPE_BF16) ? MLA_OK : MLA_E_UNSUPPORTED;
}

// A sequence's P x H query rows go to the kernels in groups of at most MLA_MAX_ROWS rows,
// one launch each, every launch reading the sequence's keys again: whole positions
// (np of them) when the heads fit in a group, otherwise slices of MLA_MAX_ROWS heads of
// one position.  A group's rows are contiguous within each sequence's rows.
struct RowGroup {
  int p0, np;  // positions p0 .. p0 + np - 1
  int h0, nh;  // heads h0 .. h0 + nh - 1
};

long row_group_count(int P, int H) {
  if ((long)P * H <= MLA_MAX_ROWS) return 1;
  if (H <= MLA_MAX_ROWS) {
    const int per = MLA_MAX_ROWS / H;
    return (P + per - 1) / per;
  }
  return (long)P * ((H + MLA_MAX_ROWS - 1) / MLA_MAX_ROWS);
}

RowGroup row_group(int P, int H, long g) {
  if ((long)P * H <= MLA_MAX_ROWS) return {0, P, 0, H};
  if (H <= MLA_MAX_ROWS) {
    const int per = MLA_MAX_ROWS / H;
    const int p0 = (int)g * per;
    return {p0, P - p0 < per ? P - p0 : per, 0, H};
  }
  const long slices = (H + MLA_MAX_ROWS - 1) / MLA_MAX_ROWS;
  const int h0 = (int)(g % slices) * MLA_MAX_ROWS;
  return {(int)(g / slices), 1, h0, H - h0 < MLA_MAX_ROWS ? H - h0 : MLA_MAX_ROWS};
}

// Groups come in at most two shapes, the first group's and the last's.
size_t workspace_bytes_all(int B, int P, int H, int max_kv_len, int num_splits, int cus) {
  const long G = row_group_count(P, H);
  size_t need = 0;
  for (long g : {0L, G - 1}) {
    const RowGroup rg = row_group(P, H, g);
    const size_t n = workspace_bytes_for(make_plan(B, rg.np, rg.nh, max_kv_len, num_splits, cus), B);
    if (n > need) need = n;
  }
  return need;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_E_INVAL: return "invalid argument";
    case MLA_E_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_E_WORKSPACE: return "workspace missing or too small";
    case MLA_E_LAUNCH: return "HIP launch or query failed";
    case MLA_E_TOO_LARGE:
      return "the call needs more scratch than mla_verify_noalloc holds "
             "(MLA_NOALLOC_SCRATCH_BYTES); use mla_verify with a workspace";
    default: return "unknown status";
  }
}

int mla_version(void) { return 100; }

int mla_decode_num_splits(int B, int P, int H, int max_kv_len, int num_splits, int num_cus) {
  if (B < 0 || P < 1 || H < 1 || max_kv_len < 0 || num_splits < 0 || num_cus < 0)
    return MLA_E_INVAL;
  if ((long)P * H > MLA_MAX_CALL_ROWS) return MLA_E_UNSUPPORTED;
  const int cus = num_cus > 0 ? num_cus : current_cu_count();
  const RowGroup rg = row_group(P, H, 0);
  return make_plan(B, rg.np, rg.nh, max_kv_len, num_splits, cus).W;
}

size_t mla_decode_workspace_size(int B, int P, int H, int max_kv_len, int num_splits) {
  if (B < 0 || P < 1 || H < 1 || max_kv_len < 0 || num_splits < 0) return 0;
  if ((long)P * H > MLA_MAX_CALL_ROWS) return 0;
  return workspace_bytes_all(B, P, H, max_kv_len, num_splits, current_cu_count());
}

namespace {

// Argument checks of mla_verify, for the whole call (before anything is launched).
mla_status check_decode(const void* q, const void* kv_cache, int kv_dtype, float kv_scale,
                        const int32_t* block_table, int max_blocks_per_seq, int block_size,
                        const int32_t* seq_lens, int B, int P, int H, int max_kv_len,
                        float softmax_scale, int num_splits) {
  if (B < 0 || P < 1 || H < 1 || max_kv_len < 0 || num_splits < 0) return MLA_E_INVAL;
  if (kv_dtype != MLA_DTYPE_BF16 && kv_dtype != MLA_DTYPE_FP8_E4M3) return MLA_E_UNSUPPORTED;
  if ((long)P * H > MLA_MAX_CALL_ROWS) return MLA_E_UNSUPPORTED;
  if (block_size <= 0 || block_size % 16 != 0 || max_blocks_per_seq < 1) return MLA_E_INVAL;
  if (!std::isfinite(softmax_scale)) return MLA_E_INVAL;
  if (kv_dtype == MLA_DTYPE_FP8_E4M3 && !finite_positive(kv_scale)) return MLA_E_INVAL;
  if (B > 0 && (!q || !kv_cache || !block_table || !seq_lens)) return MLA_E_INVAL;
  // more sequences x row blocks than counters: only the single-piece plan (no workspace)
  const RowGroup g0 = row_group(P, H, 0);  // the largest group
  if ((long)B * ((g0.np * g0.nh + 15) / 16) > MLA_MAX_COUNTERS && num_splits != 1)
    return MLA_E_UNSUPPORTED;
  if (B > 0 && current_cu_count() <= 0) return MLA_E_LAUNCH;
  return MLA_OK;
}

// Parameters of the launch over row group rg of a checked call.
void setup_decode(const void* q, const void* kv_cache, int kv_dtype, float kv_scale,
                  const int32_t* block_table, int max_blocks_per_seq, int block_size,
                  const int32_t* seq_lens, const int32_t* kv_begin, const int32_t* kv_end,
                  int B, int P, int H, const RowGroup& rg, int max_kv_len, float softmax_scale,
                  int num_splits, mla_impl::DecodeParams* p, Plan* pl) {
  const int cus = B > 0 ? current_cu_count() : 256;
  *pl = make_plan(B, rg.np, rg.nh, max_kv_len, num_splits, cus);
  const bool fp8 = kv_dtype == MLA_DTYPE_FP8_E4M3;
  const float kvs = fp8 ? kv_scale : 1.f;
  *p = mla_impl::DecodeParams{};
  p->q = static_cast<const uint16_t*>(q);
  p->kv = static_cast<const uint8_t*>(kv_cache);
  p->block_table = block_table;
  p->seq_lens = seq_lens;
  p->kv_begin = kv_begin;
  p->kv_end = kv_end;
  p->max_blocks = max_blocks_per_seq;
  p->block_size = block_size;
  p->B = B;
  p->P = rg.np;
  p->H = rg.nh;
  p->R = pl->R;
  p->RB = pl->RB;
  p->r_stride = P * H;
  p->r_off = rg.p0 * H + rg.h0;
  p->len_shift = P - rg.p0 - rg.np;
  p->W = pl->W;
  p->seg_steps = kv_dtype == MLA_DTYPE_FP8_E4M3 ? kSegmentStepsFp8 : kSegmentStepsBf16;
  p->score_scale_log2 = softmax_scale * kvs * 1.4426950408889634f;
  p->out_scale = kvs;
}

// Carve the workspace, then launch the decode kernel (and the separate merge when the
// plan needs it).  clear_counters: zero the counters the call uses first (a fill kernel
// on the same stream), for a workspace whose counters a caller cannot vouch for.
mla_status launch_verify(mla_impl::DecodeParams& p, const Plan& pl, int kv_dtype, void* out,
                         int out_dtype, float* lse, void* workspace, bool clear_counters,
                         hipStream_t stm) {
  p.out = out;
  p.out_bf16 = out_dtype == MLA_DTYPE_BF16;
  p.lse = lse;
  if (pl.W > 1) {
    const size_t rows = (size_t)(pl.W + p.B) * pl.R;
    char* ws = static_cast<char*>(workspace);
    p.counters = reinterpret_cast<int*>(ws);
    // the no-allocation entry point has nobody to read the flags: none reported
    p.flags = clear_counters ? nullptr : reinterpret_cast<int*>(ws + MLA_WORKSPACE_FLAGS_OFFSET);
    ws += kCounterBytes;
    p.part_out = reinterpret_cast<float*>(ws);
    ws += align_up(rows * MLA_HEAD_DIM_V * sizeof(float));
    p.part_lse = reinterpret_cast<float*>(ws);
    ws += align_up(rows * sizeof(float));
    p.seq_pieces = reinterpret_cast<int*>(ws);
    p.merge_in_kernel = pl.merge_in_kernel ? 1 : 0;
    if (clear_counters && p.merge_in_kernel &&
        mla_impl::launch_clear_i32(p.counters, (long)p.B * pl.RB, stm) != hipSuccess)
      return MLA_E_LAUNCH;
  } else {
    p.merge_in_kernel = 1;  // one piece: every sequence is written whole
  }
  const bool fp8 = kv_dtype == MLA_DTYPE_FP8_E4M3;
  const hipError_t e = pl.shared ? mla_impl::launch_verify_shared(p, fp8, stm)
                                 : mla_impl::launch_decode(p, fp8, stm);
  if (e != hipSuccess) return MLA_E_LAUNCH;
  if (!p.merge_in_kernel && mla_impl::launch_merge_shares(p, stm) != hipSuccess)
    return MLA_E_LAUNCH;
  return MLA_OK;
}

// ---- the entry point that allocates nothing (its scratch array is below) ----
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;

}  // namespace

// The workspace of mla_verify_noalloc: one copy per GPU, zero when the code object
// loads, held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol); it passes the per-device address
// hipGetSymbolAddress returns, looked up once per device on the first call.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of this device's copy of `scratch`, or nullptr if the runtime refuses.
void* scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

mla_status mla_verify(const void* q, const void* kv_cache, int kv_dtype, float kv_scale,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      const int32_t* seq_lens, const int32_t* kv_begin, const int32_t* kv_end,
                      int B, int P, int H, int max_kv_len, float softmax_scale, void* out,
                      int out_dtype, float* lse, int num_splits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (check_dtype_out(out_dtype) != MLA_OK) return MLA_E_UNSUPPORTED;
  if (B > 0 && !out) return MLA_E_INVAL;
  mla_status st = check_decode(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq,
                               block_size, seq_lens, B, P, H, max_kv_len, softmax_scale,
                               num_splits);
  if (st != MLA_OK) return st;
  if (B == 0) return MLA_OK;
  const size_t need = workspace_bytes_all(B, P, H, max_kv_len, num_splits, current_cu_count());
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_E_WORKSPACE;
  // row groups one after another on the stream, each leaving the counters zero
  for (long g = 0, G = row_group_count(P, H); g < G; ++g) {
    mla_impl::DecodeParams p;
    Plan pl;
    setup_decode(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq, block_size,
                 seq_lens, kv_begin, kv_end, B, P, H, row_group(P, H, g), max_kv_len,
                 softmax_scale, num_splits, &p, &pl);
    st = launch_verify(p, pl, kv_dtype, out, out_dtype, lse, workspace, false,
                       static_cast<hipStream_t>(stream));
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

mla_status mla_decode(const void* q, const void* kv_cache, int kv_dtype, float kv_scale,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      const int32_t* seq_lens, const int32_t* kv_begin, const int32_t* kv_end,
                      int B, int H, int max_kv_len, float softmax_scale, void* out,
                      int out_dtype, float* lse, int num_splits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return mla_verify(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq,
                    block_size, seq_lens, kv_begin, kv_end, B, 1, H, max_kv_len, softmax_scale,
                    out, out_dtype, lse, num_splits, workspace, workspace_bytes, stream);
}

mla_status mla_verify_noalloc(const void* q, const void* kv_cache, int kv_dtype,
                              float kv_scale, const int32_t* block_table,
                              int max_blocks_per_seq, int block_size, const int32_t* seq_lens,
                              const int32_t* kv_begin, const int32_t* kv_end, int B, int P,
                              int H, int max_kv_len, float softmax_scale, void* out,
                              int out_dtype, float* lse, int num_splits, void* stream) {
  if (check_dtype_out(out_dtype) != MLA_OK) return MLA_E_UNSUPPORTED;
  if (B > 0 && !out) return MLA_E_INVAL;
  mla_status st = check_decode(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq,
                               block_size, seq_lens, B, P, H, max_kv_len, softmax_scale,
                               num_splits);
  if (st != MLA_OK) return st;
  if (B == 0) return MLA_OK;
  const size_t need = workspace_bytes_all(B, P, H, max_kv_len, num_splits, current_cu_count());
  if (need > kScratchBytes) return MLA_E_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_for_current_device())) return MLA_E_LAUNCH;
  for (long g = 0, G = row_group_count(P, H); g < G; ++g) {
    mla_impl::DecodeParams p;
    Plan pl;
    setup_decode(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq, block_size,
                 seq_lens, kv_begin, kv_end, B, P, H, row_group(P, H, g), max_kv_len,
                 softmax_scale, num_splits, &p, &pl);
    st = launch_verify(p, pl, kv_dtype, out, out_dtype, lse, ws, true,
                       static_cast<hipStream_t>(stream));
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

mla_status mla_merge_lse(const float* part_out, const float* part_lse, int S, int N, void* out,
                         int out_dtype, float* lse, void* stream) {
  if (S < 1 || N < 0) return MLA_E_INVAL;
  if (check_dtype_out(out_dtype) != MLA_OK) return MLA_E_UNSUPPORTED;
  if (N == 0) return MLA_OK;
  if (!part_out || !part_lse || !out) return MLA_E_INVAL;
  if (mla_impl::launch_merge(part_out, part_lse, S, N, out, out_dtype == MLA_DTYPE_BF16, lse,
                             static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_E_LAUNCH;
  return MLA_OK;
}

mla_status mla_cache_write(const void* latent, long N, const int32_t* slot_mapping,
                           void* kv_cache, int kv_dtype, float kv_scale, long num_slots,
                           void* stream) {
  if (N < 0 || num_slots < 0) return MLA_E_INVAL;
  if (kv_dtype != MLA_DTYPE_BF16 && kv_dtype != MLA_DTYPE_FP8_E4M3) return MLA_E_UNSUPPORTED;
  if (kv_dtype == MLA_DTYPE_FP8_E4M3 && !finite_positive(kv_scale)) return MLA_E_INVAL;
  if (N == 0) return MLA_OK;
  if (!latent || !slot_mapping || !kv_cache) return MLA_E_INVAL;
  if (N > 0x7fffffffL / 36) return MLA_E_UNSUPPORTED;
  const hipError_t e =
      mla_impl::launch_cache_write(static_cast<const uint16_t*>(latent), N, slot_mapping,
                                   kv_cache, kv_dtype == MLA_DTYPE_FP8_E4M3, kv_scale, num_slots,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_E_LAUNCH;
}

namespace {
constexpr int kTopKListMax = 2048;  // largest k served from per-chunk candidate lists

// Workspace: candidate lists (8 bytes per entry, kTopKListMax per chunk), then one
// float per chunk for the chunk sums of rows kept whole.
size_t topk_list_bytes(int rows, int vocab) {
  return align_up((size_t)rows * (size_t)mla_impl::top_k_chunks(vocab) * kTopKListMax * 8);
}
}  // namespace

size_t mla_top_k_renorm_workspace_size(int rows, int vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  return topk_list_bytes(rows, vocab) +
         align_up((size_t)rows * (size_t)mla_impl::top_k_chunks(vocab) * 4);
}

mla_status mla_top_k_renorm_prob(const float* probs, const int32_t* top_k, int rows, int vocab,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (rows < 0) return MLA_E_INVAL;
  if (rows == 0) return MLA_OK;
  if (vocab < 1) return MLA_E_INVAL;
  if (!probs || !top_k || !out) return MLA_E_INVAL;
  const size_t need = mla_top_k_renorm_workspace_size(rows, vocab);
  if (!workspace || workspace_bytes < need || (uintptr_t)workspace % 8 != 0)
    return MLA_E_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const hipError_t e = mla_impl::launch_top_k_renorm(
      probs, top_k, rows, vocab, kTopKListMax, out, ws,
      reinterpret_cast<float*>(ws + topk_list_bytes(rows, vocab)),
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_E_LAUNCH;
}

mla_status mla_prefill(const void* q, const void* kv, int kv_dtype, float kv_scale,
                       const int32_t* cu_seqlens, int B, int T, int max_seqlen, int H,
                       float softmax_scale, void* out, int out_dtype, float* lse, void* stream) {
  if (B < 0 || T < 0 || max_seqlen < 0 || H < 1) return MLA_E_INVAL;
  if (kv_dtype != MLA_DTYPE_BF16 && kv_dtype != MLA_DTYPE_FP8_E4M3) return MLA_E_UNSUPPORTED;
  if (check_dtype_out(out_dtype) != MLA_OK) return MLA_E_UNSUPPORTED;
  if ((long)T * H > 0x7fffffffL) return MLA_E_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return MLA_E_INVAL;
  if (kv_dtype == MLA_DTYPE_FP8_E4M3 && !finite_positive(kv_scale)) return MLA_E_INVAL;
  if (B == 0 || T == 0) return MLA_OK;
  if (!q || !kv || !cu_seqlens || !out) return MLA_E_INVAL;
  const bool fp8 = kv_dtype == MLA_DTYPE_FP8_E4M3;
  const float kvs = fp8 ? kv_scale : 1.f;
  mla_impl::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv);
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.T = T;
  p.H = H;
  p.max_seqlen = max_seqlen > 0 ? max_seqlen : 1;
  p.score_scale_log2 = softmax_scale * kvs * 1.4426950408889634f;
  p.out_scale = kvs;
  p.out = out;
  p.out_bf16 = out_dtype == MLA_DTYPE_BF16;
  p.lse = lse;
  const hipError_t e = mla_impl::launch_prefill(p, fp8, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return MLA_E_UNSUPPORTED;
  return e == hipSuccess ? MLA_OK : MLA_E_LAUNCH;
}

}  // extern "C"
