// gfx950_device.h -- small device helpers shared by the prefill kernels of
// libattn.so (cross-lane swaps, buffer resources, LDS-only barriers and the
// transposing LDS read).  Not installed; not part of the ABI.
#pragma once

#include "attn_internal.h"

namespace attn {
namespace dev {

typedef short short4_t __attribute__((ext_vector_type(4)));

// max / sum of x over lanes l and l ^ 32 (both halves end with the same value)
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A raw buffer resource over [p, p + bytes).  The base address goes through
// readfirstlane so the descriptor lives in SGPRs (it is workgroup-uniform; a
// VGPR descriptor would turn every load into a waterfall loop).  Loads at
// offsets outside the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Buffer load of 16 bytes per lane straight into LDS: lane i's bytes land at
// LDS byte address lds_addr + 16 * i (one contiguous 1 KB block per
// wavefront; lds_addr is uniform).  Completion is counted by vmcnt.
__device__ __forceinline__ void buffer_load16_lds_at(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int offset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds_addr, 16, offset, 0,
                                           0, 0);
}

// s_waitcnt vmcnt(0): every buffer load of this wavefront, the copies into
// LDS among them, has landed (lgkmcnt and expcnt left at their maximum)
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): at most N of this wavefront's vector memory
// operations outstanding (they complete in issue order)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses only.  The wavefronts of a
// workgroup exchange data through LDS alone, so the barrier need not wait for
// outstanding global loads or stores (__syncthreads() does: its workgroup
// fence covers global memory too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier with no memory fence, for points where each wavefront
// has already waited for what the others will read (its copies into LDS by
// vmcnt, its LDS reads by using their results).  A fenced barrier would also
// wait for every store and load still in flight (copies into LDS count on
// vmcnt, so the memory model makes a fence on LDS wait for all of them).
// The empty asm keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void plain_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 4 fp16 values through the transposing LDS read: in each 16-lane group,
// lanes 4j..4j+3 read 16 consecutive halfs of row j and lane i receives
// column i of rows 0..3.
__device__ __forceinline__ short4_t lds_read_tr(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
}

// Lane offset (halfs) of the transposed V read in a V tile of row stride
// VROW: 16-lane group G = lane/16 covers dims 16*(G%2)..+15 of keys
// 4*hf + (lane%16)/4, four dims per lane.  Two such reads, 8 keys apart,
// form the PV operand V^T[32 dims x 16 keys]: dims dt*32 + l%32, keys
// 16c + 4*hf + (0..3) then 16c + 8 + 4*hf + (0..3) -- the key order of the
// B operand taken straight from an S^T accumulator.
template <int VROW>
__device__ __forceinline__ int pv_lane_offset(int lane) {
  const int hf = lane >> 5;
  return (4 * hf + (lane & 15) / 4) * VROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

}  // namespace dev
}  // namespace attn
