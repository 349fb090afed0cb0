// mla_api.cpp -- the C-ABI entry points declared in include/mla.h.
//
// Host work only: argument checks (before any launch), the split-KV planner,
// the workspace carve-up and the kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla.h"
#include "mla_kernels.h"

namespace {

constexpr int kStepTokens = 64;       // tokens one work-group consumes per round (4 waves x 16)
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
  int R, RB, S, chunk;
};

// Split plan.  Work-groups = B * RB * S; aim for a few per CU so long
// histories spread over the whole chip and short ones still fill it, with every
// split a whole number of 64-token rounds.  The last split takes any keys past
// S * chunk, so a wrong max_kv_len hint costs time, never correctness.
Plan make_plan(int B, int P, int H, int max_kv_len, int num_splits, int cus) {
  Plan pl;
  pl.R = P * H;
  pl.RB = (pl.R + 15) / 16;
  const long len = max_kv_len > 0 ? max_kv_len : 1;
  const long rounds = (len + kStepTokens - 1) / kStepTokens;
  long S;
  if (num_splits > 0) {
    S = num_splits;
  } else {
    const int target = 2 * (cus > 0 ? cus : 256);
    const long units = (long)(B > 0 ? B : 1) * pl.RB;
    S = (target + units - 1) / units;
    if (S > rounds) S = rounds;
    if (S < 1) S = 1;
  }
  long chunk_rounds = (rounds + S - 1) / S;
  pl.chunk = (int)(chunk_rounds * kStepTokens);
  if (num_splits <= 0) S = (rounds + chunk_rounds - 1) / chunk_rounds;
  pl.S = (int)S;
  return pl;
}

size_t workspace_bytes_for(const Plan& pl, int B) {
  if (pl.S <= 1) return 0;
  const size_t rows = (size_t)pl.S * B * pl.R;
  return align_up(rows * MLA_HEAD_DIM_V * sizeof(float)) + align_up(rows * sizeof(float));
}

bool finite_positive(float x) { return std::isfinite(x) && x > 0.f; }

mla_status check_dtype_out(int out_dtype) {
  return (out_dtype == MLA_DTYPE_FP32 || out_dtype == MLA_DTYPE_BF16) ? MLA_OK : MLA_E_UNSUPPORTED;
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
    default: return "unknown status";
  }
}

int mla_version(void) { return 100; }

int mla_decode_num_splits(int B, int P, int H, int max_kv_len, int num_splits, int num_cus) {
  if (B < 0 || P < 1 || H < 1 || max_kv_len < 0 || num_splits < 0 || num_cus < 0)
    return MLA_E_INVAL;
  if ((long)P * H > MLA_MAX_ROWS) return MLA_E_UNSUPPORTED;
  const int cus = num_cus > 0 ? num_cus : current_cu_count();
  return make_plan(B, P, H, max_kv_len, num_splits, cus).S;
}

size_t mla_decode_workspace_size(int B, int P, int H, int max_kv_len, int num_splits) {
  if (B < 0 || P < 1 || H < 1 || max_kv_len < 0 || num_splits < 0) return 0;
  if ((long)P * H > MLA_MAX_ROWS) return 0;
  return workspace_bytes_for(make_plan(B, P, H, max_kv_len, num_splits, current_cu_count()), B);
}

namespace {

// Shared argument checks and parameter setup of mla_verify / mla_verify_partials.
mla_status setup_decode(const void* q, const void* kv_cache, int kv_dtype, float kv_scale,
                        const int32_t* block_table, int max_blocks_per_seq, int block_size,
                        const int32_t* seq_lens, const int32_t* kv_begin, const int32_t* kv_end,
                        int B, int P, int H, int max_kv_len, float softmax_scale,
                        int num_splits, mla_impl::DecodeParams* p, Plan* pl) {
  if (B < 0 || P < 1 || H < 1 || max_kv_len < 0 || num_splits < 0) return MLA_E_INVAL;
  if (kv_dtype != MLA_DTYPE_BF16 && kv_dtype != MLA_DTYPE_FP8_E4M3) return MLA_E_UNSUPPORTED;
  if ((long)P * H > MLA_MAX_ROWS) return MLA_E_UNSUPPORTED;
  if (block_size <= 0 || block_size % 16 != 0 || max_blocks_per_seq < 1) return MLA_E_INVAL;
  if (!std::isfinite(softmax_scale)) return MLA_E_INVAL;
  if (kv_dtype == MLA_DTYPE_FP8_E4M3 && !finite_positive(kv_scale)) return MLA_E_INVAL;
  if (B > 0 && (!q || !kv_cache || !block_table || !seq_lens)) return MLA_E_INVAL;
  const int cus = B > 0 ? current_cu_count() : 256;
  if (cus <= 0) return MLA_E_LAUNCH;
  *pl = make_plan(B, P, H, max_kv_len, num_splits, cus);
  if (pl->S > 0 && (long)B * pl->S > 0x3fffffffL / (8 * pl->RB)) return MLA_E_UNSUPPORTED;
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
  p->P = P;
  p->H = H;
  p->R = pl->R;
  p->RB = pl->RB;
  p->S = pl->S;
  p->chunk_tokens = pl->chunk;
  p->pairs = B * pl->S;
  p->score_scale_log2 = softmax_scale * kvs * 1.4426950408889634f;
  p->out_scale = kvs;
  return MLA_OK;
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
  mla_impl::DecodeParams p;
  Plan pl;
  mla_status st = setup_decode(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq,
                               block_size, seq_lens, kv_begin, kv_end, B, P, H, max_kv_len,
                               softmax_scale, num_splits, &p, &pl);
  if (st != MLA_OK) return st;
  if (B == 0) return MLA_OK;
  const size_t need = workspace_bytes_for(pl, B);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_E_WORKSPACE;
  p.out = out;
  p.out_bf16 = out_dtype == MLA_DTYPE_BF16;
  p.lse = lse;
  const int N = B * pl.R;
  if (pl.S > 1) {
    char* ws = static_cast<char*>(workspace);
    p.part_out = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(
        ws + align_up((size_t)pl.S * N * MLA_HEAD_DIM_V * sizeof(float)));
  }
  hipStream_t stm = static_cast<hipStream_t>(stream);
  const bool fp8 = kv_dtype == MLA_DTYPE_FP8_E4M3;
  if (mla_impl::launch_decode_partial(p, fp8, stm) != hipSuccess) return MLA_E_LAUNCH;
  if (pl.S > 1 &&
      mla_impl::launch_merge(p.part_out, p.part_lse, pl.S, N, out, p.out_bf16, lse, stm) !=
          hipSuccess)
    return MLA_E_LAUNCH;
  return MLA_OK;
}

mla_status mla_verify_partials(const void* q, const void* kv_cache, int kv_dtype, float kv_scale,
                               const int32_t* block_table, int max_blocks_per_seq,
                               int block_size, const int32_t* seq_lens, const int32_t* kv_begin,
                               const int32_t* kv_end, int B, int P, int H, int max_kv_len,
                               float softmax_scale, int num_splits, float* part_out,
                               float* part_lse, void* stream) {
  if (B > 0 && (!part_out || !part_lse)) return MLA_E_INVAL;
  mla_impl::DecodeParams p;
  Plan pl;
  mla_status st = setup_decode(q, kv_cache, kv_dtype, kv_scale, block_table, max_blocks_per_seq,
                               block_size, seq_lens, kv_begin, kv_end, B, P, H, max_kv_len,
                               softmax_scale, num_splits, &p, &pl);
  if (st != MLA_OK) return st;
  if (B == 0) return MLA_OK;
  if (pl.S == 1) {  // one split: the kernel writes its normalised rows directly
    p.out = part_out;
    p.out_bf16 = 0;
    p.lse = part_lse;
  } else {
    p.part_out = part_out;
    p.part_lse = part_lse;
  }
  const bool fp8 = kv_dtype == MLA_DTYPE_FP8_E4M3;
  if (mla_impl::launch_decode_partial(p, fp8, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_E_LAUNCH;
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

mla_status mla_prefill(const void* q, const void* kv, int kv_dtype, float kv_scale,
                       const int32_t* cu_seqlens, int B, int T, int max_seqlen, int H,
                       float softmax_scale, void* out, int out_dtype, float* lse, void* stream) {
  if (B < 0 || T < 0 || max_seqlen < 0 || H < 1) return MLA_E_INVAL;
  if (kv_dtype != MLA_DTYPE_BF16 && kv_dtype != MLA_DTYPE_FP8_E4M3) return MLA_E_UNSUPPORTED;
  if (check_dtype_out(out_dtype) != MLA_OK) return MLA_E_UNSUPPORTED;
  if (H > MLA_MAX_ROWS) return MLA_E_UNSUPPORTED;
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
