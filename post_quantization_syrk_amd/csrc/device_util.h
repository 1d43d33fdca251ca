// Device helpers shared by the engine's gfx950 kernels (not part of the C ABI): raw buffer
// access with per-lane masking, s_waitcnt immediates and the workgroup barrier used to hand
// LDS tiles from the copy stage to the MFMA stage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer access with per-lane masking: a lane whose byte offset lies at or past the
// descriptor's record count reads 0 and its store is dropped, so the masked loads and stores
// at a tile's edge need no branches (a branch around an access makes the compiler wait for
// every memory operation in flight where the paths join).  0x00020000 is the descriptor's
// data-format word on gfx9.
constexpr int OOB = 0x7ffffff0;   // the record count of an unbounded descriptor

// Descriptor over `bytes` bytes at base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Descriptor whose only masked offsets are those at or past OOB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return rsrc(base, OOB);
}
__device__ __forceinline__ float4 bload4(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bstore(float v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]):
// wait until at most n vector-memory operations are outstanding, or until no LDS/scalar one is.
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int WAIT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Workgroup barrier for LDS hand-off; also a hard boundary for the instruction scheduler.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace
}  // namespace kq
