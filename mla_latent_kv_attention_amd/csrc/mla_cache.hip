// mla_cache.hip -- latent-row cache write for gfx950: quantise new positions' rows
// and scatter them into their paged cache slots.
//
// Every cached position holds one 576-wide latent row (512 latent + 64 rotary
// values), 576 bytes per position in FP8 (Kimi K3 engineering report, section
// "缓存可复用，还要能一致地恢复"); FP8 latent caches are what the FP8 KV decode
// paths read (InferenceX blog on Kimi K2.5, section "PR #35850 修复了什么").  A
// BF16 cache receives the rows unchanged; an FP8 cache receives, per value x,
// the OCP E4M3FN code nearest to fp32(x / kv_scale) clamped to +-448, ties to
// the even mantissa, NaN as 0x7F -- the value the decode kernels multiply back
// by kv_scale.
//
// One thread per 16-value chunk of a row (36 chunks per row): two 16-byte loads
// of BF16, one 16-byte store of FP8 codes (or two of BF16).  Consecutive threads
// take consecutive chunks, so a wave reads and writes contiguous runs.  The op is
// HBM-bound: 1,152 bytes in and 576 (FP8) or 1,152 (BF16) bytes out per row.  The
// stores carry the nontemporal hint (32,768 rows into an FP8 cache: 13.8 -> 13.0 us;
// on the loads the hint was slower).
#include <cmath>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla_impl {
using namespace mla_dev;

namespace {

constexpr int kChunks = kDK / 16;  // 36 chunks of 16 values per row

// E4M3FN code of fp32 y, round to nearest even, saturating at 448, NaN -> 0x7F.
// Normal range: round the fp32 significand to 3 fraction bits at bit 20 (a carry
// into the exponent is the correct result); below 2^-6 the code is the number of
// 2^-9 steps, rounded to nearest even.
__device__ __forceinline__ uint32_t fp8_e4m3fn_code(float y) {
  if (y != y) return 0x7Fu;
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);  // 0 .. 8; 8 is the code of 2^-6
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);  // exponent bias 127 -> 7
  }
  return code | sign;
}

// fp32(x / s), correctly rounded, from r = fp32(1 / s) and one fused correction: the
// product y0 = x * r is within an ulp of x / s, the residual x - s * y0 is exact in an
// fma, and y0 + r * residual rounded once is the correctly rounded quotient when
// nothing underflows or overflows (Markstein's theorem on division by a correctly
// rounded reciprocal).  The code only depends on the exact quotient between 2^-10 and
// 448, so the correction is applied where |y0| >= 2^-100 and y0 is finite: below that
// y0 carries x's sign and codes to a signed zero (where the correction could cancel to
// +0), and an infinite y0 saturates like the infinite or huge x / s.  Three or four
// instructions instead of a division.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float y0 = x * r;
  const float e = __builtin_fmaf(-s, y0, x);
  const bool correct = __builtin_fabsf(y0) >= 0x1p-100f && __builtin_isfinite(y0);
  return correct ? __builtin_fmaf(e, r, y0) : y0;
}

// kFastDiv: the quotient through div_by_scale, for scales whose reciprocal is a normal
// fp32 number (the host checks); otherwise a correctly rounded division per value.
template <bool kFp8, bool kFastDiv>
__global__ __launch_bounds__(256) void cache_write_kernel(const uint16_t* __restrict__ latent,
                                                          long N, const int32_t* __restrict__ slot,
                                                          uint8_t* __restrict__ kv,
                                                          float kv_scale, long num_slots) {
  const long item = (long)blockIdx.x * 256 + threadIdx.x;
  if (item >= N * kChunks) return;
  const long n = item / kChunks;
  const int c = (int)(item - n * kChunks);
  const long s = slot[n];
  if (s < 0 || s >= num_slots) return;  // padding positions, or outside the cache
  const uint16_t* src = latent + n * kDK + 16 * c;
  const u32x4 lo = *(const u32x4*)src;
  const u32x4 hi = *(const u32x4*)(src + 8);
  if constexpr (kFp8) {
    const float r = __fdiv_rn(1.f, kv_scale);
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t pair = w[2 * q + h];
        const float x0 = __uint_as_float(pair << 16);          // BF16 -> fp32, exact
        const float x1 = __uint_as_float(pair & 0xFFFF0000u);
        const float y0 = kFastDiv ? div_by_scale(x0, kv_scale, r) : __fdiv_rn(x0, kv_scale);
        const float y1 = kFastDiv ? div_by_scale(x1, kv_scale, r) : __fdiv_rn(x1, kv_scale);
        word |= fp8_e4m3fn_code(y0) << (16 * h);
        word |= fp8_e4m3fn_code(y1) << (16 * h + 8);
      }
      out[q] = word;
    }
    __builtin_nontemporal_store(out, (u32x4*)(kv + s * kDK + 16 * c));
  } else {
    uint16_t* dst = (uint16_t*)kv + s * kDK + 16 * c;
    __builtin_nontemporal_store(lo, (u32x4*)dst);
    __builtin_nontemporal_store(hi, (u32x4*)(dst + 8));
  }
}

}  // namespace

hipError_t launch_cache_write(const uint16_t* latent, long N, const int32_t* slot, void* kv,
                              bool kv_fp8, float kv_scale, long num_slots, hipStream_t stream) {
  const long items = N * kChunks;
  if (items == 0) return hipSuccess;
  const long blocks = (items + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const float r = 1.f / kv_scale;  // IEEE division on the host: fp32(1 / kv_scale)
  const bool fast = std::isnormal(r);
  if (kv_fp8 && fast)
    hipLaunchKernelGGL((cache_write_kernel<true, true>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, latent, N, slot, (uint8_t*)kv, kv_scale, num_slots);
  else if (kv_fp8)
    hipLaunchKernelGGL((cache_write_kernel<true, false>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, latent, N, slot, (uint8_t*)kv, kv_scale, num_slots);
  else
    hipLaunchKernelGGL((cache_write_kernel<false, false>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, latent, N, slot, (uint8_t*)kv, kv_scale, num_slots);
  return hipGetLastError();
}

}  // namespace mla_impl
