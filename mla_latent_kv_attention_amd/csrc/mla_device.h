// mla_device.h -- gfx950 device helpers shared by the MLA kernels.
//
// Register-fragment layouts below were checked on gfx950 hardware: for the
// 16x16xK bf16 MFMA with K/16 values per lane, lane l holds A[l % 16][(K/4) *
// (l / 16) + i], B[(K/4) * (l / 16) + i][l % 16], and the 16x16 f32 result
// C[4 * (l / 16) + i][l % 16].  The LDS transpose read ds_read_b64_tr_b16
// works on 16-lane groups: lane j of a group receives element (j % 4) of the
// 8-byte chunk addressed by lane (4 * s + j / 4), for s = 0..3.  Its 8-bit form
// ds_read_b64_tr_b8 likewise: lane j of a group receives byte j % 8 of the chunk
// addressed by lane (2 * s + j / 8), for s = 0..7, i.e. the group's 8 chunk pairs
// are 8 rows of 16 bytes and lane j gets column j of all 8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDK = 576;  // key width (512 latent + 64 rotary)
constexpr int kDV = 512;  // value width (the latent part)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// S += A (16 x 32) * B (32 x 16), bf16 in, fp32 accumulate.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// C += A (16 x 16) * B (16 x 16), bf16 in (as raw 16-bit lanes), fp32 accumulate.
__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposed 4 x 16-bit LDS read (see the layout note at the top).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Transposed 8 x 8-bit LDS read (see the layout note at the top).
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p)));
}

// Exact OCP E4M3FN -> bf16 for four codes packed in one dword (bytes 0..3).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

// 8 FP8 codes -> bf16x8, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  bf16x2 p0, p1, p2, p3;
  fp8x4_to_bf16(w.x, p0, p1);
  fp8x4_to_bf16(w.y, p2, p3);
  return (bf16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 16 FP8 codes -> two bf16x8 (codes 0..7, codes 8..15), exact.
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 w, bf16x8& a, bf16x8& b) {
  bf16x2 p0, p1, p2, p3, p4, p5, p6, p7;
  fp8x4_to_bf16(w.x, p0, p1);
  fp8x4_to_bf16(w.y, p2, p3);
  fp8x4_to_bf16(w.z, p4, p5);
  fp8x4_to_bf16(w.w, p6, p7);
  a = (bf16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  b = (bf16x8){p4.x, p4.y, p5.x, p5.y, p6.x, p6.y, p7.x, p7.y};
}

// x *= s for MFMA accumulator values kept in AGPRs: each element is read into a
// VGPR, scaled and written back, so the accumulator keeps its register class
// across a loop (a plain VALU multiply on it makes the compiler carry every
// accumulator value through VGPRs on every iteration).
template <int kN>
__device__ __forceinline__ void scale_agpr(float __attribute__((ext_vector_type(kN)))& acc,
                                           float s) {
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    float x = acc[i];
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(s));
    acc[i] = x;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Lane pairs {l, l ^ 32} and {l, l ^ 16} through the gfx950 VALU lane swaps
// (no LDS round trip).  permlane32_swap(a, b) exchanges lanes 32-63 of a with
// lanes 0-31 of b; with a = b = v the two results hold v[l & 31] and
// v[(l & 31) + 32].  permlane16_swap does the same for odd / even 16-lane rows.
__device__ __forceinline__ void xor32_pair(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void xor16_pair(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max16x4(float v) {
  // max over lanes {l, l ^ 16, l ^ 32, l ^ 48}
  float a, b;
  xor16_pair(v, a, b);
  v = fmaxf(a, b);
  xor32_pair(v, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_sum16x4(float v) {
  float a, b;
  xor16_pair(v, a, b);
  v = a + b;
  xor32_pair(v, a, b);
  return a + b;
}

__device__ __forceinline__ float wave_max_xor32(float v) {
  float a, b;
  xor32_pair(v, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_sum_xor32(float v) {
  float a, b;
  xor32_pair(v, a, b);
  return a + b;
}

// Keep the compiler from moving LDS accesses across this point; lanes of one
// wave exchange data through LDS around it.
// Agent-coherent global accesses without fences.  On gfx950 the L2 is per XCD;
// a relaxed agent-scope atomic store or load is issued with the sc1 cache bit,
// which writes through to / reads from the device-coherent level, while a
// release or acquire fence would write back or invalidate the whole XCD's L2.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-coherent accesses through a buffer resource: `base` is uniform
// across the wave, `off` a per-lane byte offset (raw buffer, 2^31 - 1 bytes).
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t agent_rsrc(float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ f32x4 load_agent16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicySc1));
}
__device__ __forceinline__ void store_agent16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCachePolicySc1);
}

// Wait until every vector memory access this wave issued has completed (for
// stores: acknowledged at the level their cache bits name).  The signal fences
// keep the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_vm_all() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt = 0, other counters free
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Inclusive prefix sum over the 64 lanes of a wave: a Hillis-Steele scan within each
// row of 16 lanes through DPP row shifts (register-to-register, no LDS round trip),
// then the totals of the rows below added from lanes 15, 31 and 47.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                 r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
}

// One 16-byte global -> LDS copy per lane, no VGPR staging: lane l reads base + voff
// (base uniform, voff per lane) and lands at LDS byte lds_base + 16 l.  Issued through
// asm so that the compiler does not fence every later LDS read behind all outstanding
// loads (it would put a full vmcnt(0) before each); the caller waits for its own copies
// with explicit vmcnt waits and a barrier.  The LDS base goes in M0 as an operand of the
// asm ("{m0}"), so the compiler sets M0 itself and knows the asm reads it: nothing
// writes M0 behind its back.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// The same copy from a full 64-bit address per lane.
__device__ __forceinline__ void dma16_addr(const void* src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their no-wait maxima).
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(kN >= 0 && kN < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Phase stamps of the timeline build (libmla_timeline.so, compiled with MLA_TIMELINE):
// the first thread of work-group g writes the 100 MHz real-time counter at phase
// boundary s to buf[g * kStampSlots + s], for the first kStampGroups work-groups.  The
// stores are thread 0's only and come after (never between) the copies whose waits
// count outstanding operations, so they can only make those waits stricter.  Every
// other build compiles the stamps out.
constexpr int kStampGroups = 4096;
constexpr int kStampSlots = 8;

}  // namespace mla_dev

#ifdef MLA_TIMELINE
#define MLA_STAMP(buf, s)                                                           \
  do {                                                                              \
    if (threadIdx.x == 0 && blockIdx.x < mla_dev::kStampGroups)                     \
      (buf)[blockIdx.x * mla_dev::kStampSlots + (s)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define MLA_STAMP(buf, s) \
  do {                    \
  } while (0)
#endif
