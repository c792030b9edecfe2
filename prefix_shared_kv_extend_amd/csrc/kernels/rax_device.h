// Device-side helpers shared by librax's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace raxk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Device error word: bits of RAX_DEVERR_* for indices a kernel skipped.
extern __device__ int32_t g_rax_err;

__device__ __forceinline__ void flag_error(int32_t bit) { atomicOr(&g_rax_err, bit); }

// Workgroup ids are dispatched round-robin over the 8 XCDs (each with its own L2).
// Map the linear id so that ids landing on one XCD form contiguous runs of work items,
// i.e. work items that share K/V tiles run under the same L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  constexpr int64_t kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  const int64_t per = nblocks / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds wave-uniform).
// Written as asm so that the compiler, which cannot tell which LDS bytes such a load
// writes, does not wait for every one in flight before each later LDS read: the kernel
// waits for them itself (s_waitcnt vmcnt, in issue order).
__device__ __forceinline__ void lds_load16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// 4 bytes per lane from global memory into LDS at lds + 4 * lane (lds wave-uniform).
__device__ __forceinline__ void lds_load4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// The same load with the non-temporal hint, for rows read once per call: measured on a
// 4 GB streaming read, plain 16-byte loads reach ~5.8 TB/s and non-temporal ones ~7.2 TB/s
// (the lines are not kept in the caches on the way).
__device__ __forceinline__ void lds_load16_nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds) : "memory", "m0");
}

// Wait until at most N of this wave's vector memory loads are in flight (they retire in
// issue order). vmcnt is bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) not waited for.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Cross-lane exchanges in the VALU (gfx950): v_permlane32_swap swaps lanes 32..63 of its
// first register with lanes 0..31 of its second, v_permlane16_swap the odd 16-lane rows of
// its first register with the even rows of its second. Written as asm: this toolchain's
// builtins hand back the first register for both results. The s_nops pad the hazards
// between a VALU write and the swap's read, and the swap's write and a later read.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// x combined (max or sum) with its value in lane l ^ 32, and in lane l ^ 16: after a swap
// of two copies of x, lane l of the two registers holds x[l] and x[l ^ 32] (or ^ 16), in
// some order.
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  return a + b;
}
__device__ __forceinline__ float max_xor16(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor16(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  return a + b;
}

// Stores and loads coherent at device scope (relaxed atomics: on gfx950 they carry the sc1
// bit and pass through the XCD's L2), for data that another workgroup of the same launch,
// possibly on another XCD, reads after a device-scope atomic has ordered the two.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-uniform copy (kept in an SGPR) of a value that is the same in every lane.
__device__ __forceinline__ uint32_t uni32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Byte address in LDS of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

}  // namespace raxk
