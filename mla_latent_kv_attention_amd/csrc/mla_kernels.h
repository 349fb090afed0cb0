// mla_kernels.h -- launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla_impl {

// Decode / verify over a paged latent cache in one persistent launch: the
// batch's key ranges, cut into 16-token steps and concatenated, are divided into
// W equal pieces; work-group (piece w, 16-row block rb) walks the sequence
// segments of its piece, and the last piece to finish a sequence merges that
// sequence's partials.
struct DecodeParams {
  const uint16_t* q;           // [B, r_stride, 576] bf16; this launch's rows: R = P * H
  const uint8_t* kv;           // [num_blocks, block_size, 576] bf16 or fp8 codes
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* seq_lens;     // [B]
  const int32_t* kv_begin;     // [B] or null
  const int32_t* kv_end;       // [B] or null
  int max_blocks;
  int block_size;              // multiple of 16
  int B, P, H, R, RB;          // RB = ceil(R / 16)
  // A sequence of more than 64 query rows runs as several launches, each over a group of
  // at most 64 of its rows (whole positions, or 64-head slices of one position):
  int r_stride;                // rows per sequence in q, out and lse (the call's P * H)
  int r_off;                   // this launch's first row within each sequence's rows
  int len_shift;               // its last position is this many before the sequence's last
  int W;                       // pieces of the concatenated step list
  int seg_steps;               // virtual steps charged per sequence a piece touches
  float score_scale_log2;      // softmax_scale * kv_scale * log2(e)
  float out_scale;             // kv_scale for fp8 caches, 1 for bf16
  float* part_out;             // [W + B, R, 512]: slot w + b holds piece w's share of sequence b
  float* part_lse;             // [W + B, R]
  int* counters;               // [B, RB] (B * RB <= MLA_MAX_COUNTERS): zero on entry, left zero
  int* flags;                  // error flags (MLA_FLAG_*), ORed in; null: not reported
  int merge_in_kernel;         // 1: the last piece of a sequence merges; 0: launch_merge_shares
  int* seq_pieces;             // [B, 2]: first and last piece of each sequence (merge_in_kernel 0)
  void* out;                   // [B * r_stride, 512] fp32 or bf16
  int out_bf16;
  float* lse;                  // [B * r_stride] or null
};

// The same for sequences of 2 to 4 row blocks: one work-group per piece serves them all
// (grid W), each latent row read once per piece and staged in LDS.
hipError_t launch_verify_shared(const DecodeParams& p, bool kv_fp8, hipStream_t stream);

// Work-groups launch_decode uses for W pieces and RB row blocks.
int decode_grid_size(int W, int RB);

hipError_t launch_decode(const DecodeParams& p, bool kv_fp8, hipStream_t stream);

// Zero n int32 values at p with a fill kernel (no memset node under graph capture).
hipError_t launch_clear_i32(int* p, long n, hipStream_t stream);

// The separate merge of a launch_decode with merge_in_kernel = 0 (same params).
hipError_t launch_merge_shares(const DecodeParams& p, hipStream_t stream);

hipError_t launch_merge(const float* part_out, const float* part_lse, int S, int N, void* out,
                        int out_bf16, float* lse, hipStream_t stream);

// Quantise (FP8) or copy (BF16) N latent rows into cache slots slot[n] of a cache
// with num_slots rows; slots outside [0, num_slots) are skipped.
hipError_t launch_cache_write(const uint16_t* latent, long N, const int32_t* slot, void* kv,
                              bool kv_fp8, float kv_scale, long num_slots, hipStream_t stream);

// Top-k renormalisation of rows x vocab fp32 probabilities (two launches).  The
// list buffer holds rows * top_k_chunks(vocab) * list_max entries of 8 bytes, sums
// rows * top_k_chunks(vocab) floats.
long top_k_chunks(int vocab);
hipError_t launch_top_k_renorm(const float* probs, const int32_t* top_k, int rows, int vocab,
                               int list_max, float* out, void* list, float* sums,
                               hipStream_t stream);

struct PrefillParams {
  const uint16_t* q;           // [T, H, 576]
  const uint8_t* kv;           // [T, 576] bf16 or fp8 codes
  const int32_t* cu_seqlens;   // [B + 1]
  int B, T, H, max_seqlen;
  float score_scale_log2;
  float out_scale;
  void* out;                   // [T, H, 512]
  int out_bf16;
  float* lse;                  // [T, H] or null
};

hipError_t launch_prefill(const PrefillParams& p, bool kv_fp8, hipStream_t stream);

}  // namespace mla_impl
