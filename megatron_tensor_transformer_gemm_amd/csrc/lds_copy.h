// Asynchronous HBM/L2 -> LDS copies for gfx950 kernels (internal).
//
// buffer_load_dwordx4 ... lds moves 16 bytes per lane straight into LDS at M0 + 16*lane,
// without staging registers.  A lane whose offset is at or beyond the descriptor's
// num_records reads zeros, so ragged edges need no separate code: masked lanes pass kOOB.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

constexpr uint32_t kOOB = 0x40000000u;       // voffset of a masked lane: >= num_records
constexpr int kNumRecords = 0x40000000;      // every valid per-lane offset is below 1 GiB
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data format (gfx9 family)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor as four SGPRs (base must be wave-uniform).
__device__ __forceinline__ i32x4 make_desc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xFFFF, kNumRecords, kRsrcWord3};
}

// One buffer_load_dwordx4 ... lds: each lane copies 16 bytes from desc+voff into LDS at
// lds_base + 16*lane.  Issued as inline assembly so that the compiler does not track the
// asynchronous LDS write: completion is managed explicitly (vmcnt + barrier), which lets
// several stages stay in flight.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved, yet this asm does set it
__device__ __forceinline__ void copy16_to_lds(const i32x4& desc, uint32_t voff,
                                              uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier after this wave's copies have landed except for the newest I, and
// its LDS reads have completed.  (A __syncthreads() would also wait for every copy in
// flight: the fence it carries treats them as pending stores.)
template <int I>
__device__ __forceinline__ void sync_copies() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(I) : "memory");
}

}  // namespace tpk
