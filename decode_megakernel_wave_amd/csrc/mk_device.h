// mk_device.h -- gfx950 device primitives of the monokernel: coherent
// loads/stores for cross-workgroup sync, wavefront DPP reductions, and the
// per-wavefront LDS weight ring fed by nontemporal global->LDS loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_layout.h"

namespace mk {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));


constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- memory helpers
// Cross-workgroup traffic (sentinel polls, published outputs, counters) uses
// system-scope atomics, which gfx950 encodes with both cache-policy bits
// (sc0 sc1): the access bypasses the CU's L1 and the XCD's L2 and goes to the
// memory-side coherence point.  This is the HIP counterpart of the uncached
// read the sentinel needs ("7 - AMD et le monokernel", section 7.3): a poll
// must never be answered from a cached copy.  Agent-scope (sc1 only) loads were
// measured to keep returning a stale line on another XCD.
//
// Every pointer that reaches device memory is cast to the global address
// space (1) first, so the compiler emits global_* instead of flat_*
// instructions: flat operations also count in lgkmcnt, which would make each
// LDS barrier wait for outstanding global stores to be acknowledged.
#ifndef MK_SYNC_SCOPE
#define MK_SYNC_SCOPE __HIP_MEMORY_SCOPE_SYSTEM
#endif
#define MK_SCOPE MK_SYNC_SCOPE
#define MK_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ MK_GLOBAL T* gp(T* p) { return (MK_GLOBAL T*)p; }

__device__ __forceinline__ uint32_t ldc32(const void* p) {
  return __hip_atomic_load(gp((const uint32_t*)p), __ATOMIC_RELAXED, MK_SCOPE);
}
__device__ __forceinline__ uint16_t ldc16(const void* p) {
  return __hip_atomic_load(gp((const uint16_t*)p), __ATOMIC_RELAXED, MK_SCOPE);
}
__device__ __forceinline__ uint64_t ldc64(const void* p) {
  return __hip_atomic_load(gp((const uint64_t*)p), __ATOMIC_RELAXED, MK_SCOPE);
}
__device__ __forceinline__ void stc32(void* p, uint32_t v) {
  __hip_atomic_store(gp((uint32_t*)p), v, __ATOMIC_RELAXED, MK_SCOPE);
}
__device__ __forceinline__ void stc16(void* p, uint16_t v) {
  __hip_atomic_store(gp((uint16_t*)p), v, __ATOMIC_RELAXED, MK_SCOPE);
}
__device__ __forceinline__ void stc64(void* p, uint64_t v) {
  __hip_atomic_store(gp((uint64_t*)p), v, __ATOMIC_RELAXED, MK_SCOPE);
}
__device__ __forceinline__ void stcf(float* p, float v) { stc32(p, __float_as_uint(v)); }

// 16 bytes of sync words per request: a buffer load with the same cache-policy
// bits as the system-scope loads above (sc0 sc1), marked volatile (bit 31 of
// the policy operand) so the compiler re-issues it in every poll round.  Each
// aligned 4-byte word of the result is read whole, so a reader checks every
// word for the sentinel, as it would after four single loads; the gain is a
// quarter of the requests in flight while hundreds of workgroups poll.  The
// buffer resource bounds the access: bytes beyond `bytes` read as zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
#if MK_SYNC_SCOPE == __HIP_MEMORY_SCOPE_SYSTEM
constexpr int kPolicySync = (int)(0x80000000u | 1u | 16u);  // volatile | sc0 | sc1
#else
constexpr int kPolicySync = (int)(0x80000000u | 16u);       // volatile | sc1
#endif
__device__ __forceinline__ Rsrc sync_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u4 ldc128(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kPolicySync));
}
__device__ __forceinline__ u2 ldc64v(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kPolicySync));
}

// Release / acquire between workgroups for data whose arrival the reader
// cannot see in the data itself (the KV cache and the sentinel re-arms at a
// step boundary; every stage in counter mode).  Everything the kernel shares
// between workgroups is written with the system-scope stores above, which
// the L2 writes through and acknowledges once they are visible at the
// coherence point, and read with system-scope loads or, for the KV cache of
// earlier positions, with plain loads of lines no cache can hold stale (a
// line is never read before it is written in a launch, and every launch
// starts by invalidating its caches).  So a release only has to wait for the
// wavefront's stores to be acknowledged, and an acquire only has to keep the
// compiler from moving later loads above the poll.  Building with
// MK_FULL_FENCES selects the agent-scope fences instead (L2 write-back and
// invalidation), the conservative reading of the memory model.
__device__ __forceinline__ void stores_acked() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
#ifdef MK_FULL_FENCES
__device__ __forceinline__ void release_stores() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_polled() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
#else
__device__ __forceinline__ void release_stores() { stores_acked(); }
__device__ __forceinline__ void acquire_polled() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }
#endif

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  uint64_t v = (uint64_t)p;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier ordering LDS traffic only: the fences name the "local"
// address space, so outstanding global loads (the weight ring) and stores
// stay in flight across it, and the compiler may keep values it loaded from
// global memory in registers (no blanket memory clobber).
__device__ __forceinline__ void cta_sync_hw() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int xcc_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 15;
}

// ---------------------------------------------------------------- wavefront reductions (DPP)
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
// Sum over the 64 lanes; the result is uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);         // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);         // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);        // row_half_mirror
  v += dpp<0x140>(v);        // row_mirror: every lane holds its 16-lane row sum
  v += dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------- weight ring
struct Ring {
  uint32_t lds;          // LDS byte address of this wavefront's ring
  const uint8_t* g;      // stream base
  uint32_t n;            // chunks per step
  uint32_t issue;        // next chunk (mod n) to request
  uint32_t slot;         // ring slot holding the next chunk to consume
  uint32_t owed;         // slots read but not yet refilled (the `owed` slots before `slot`)
};

// The ring is touched only through inline asm (the DMA that fills a slot and
// the ds_read that drains it), so none of these statements needs a "memory"
// clobber: a clobber would make the compiler reload every value it keeps in
// memory (kernel parameters, LDS pointers) after each chunk, and the next
// lgkmcnt wait would then stall on those scalar loads.  Volatile asm
// statements keep their program order relative to each other.
__device__ __forceinline__ void dma_chunk(uint32_t lds_addr, const uint8_t* g, uint32_t voff) {
  uint32_t save;
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  g = (const uint8_t*)uniform_ptr(g);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(voff), "s"(g));
}

__device__ __forceinline__ void ring_start(Ring& r) {
  if (r.n == 0) return;
  const uint32_t lane16 = lane_id() * 16;
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    dma_chunk(r.lds + i * 1024, r.g, r.issue * 1024 + lane16);
    r.issue = (r.issue + 1 == r.n) ? 0 : r.issue + 1;
  }
  r.slot = 0;
}

// Read N ring chunks (N <= 4) at LDS addresses a[] after waiting for
// vmcnt(W), with one LDS wait; one asm block, so no use of v[] can be
// scheduled before the data is there.
template <int N, int W>
__device__ __forceinline__ void ring_load(const uint32_t (&a)[4], u4 (&v)[4]) {
  if constexpr (N == 1) {
    asm volatile("s_waitcnt vmcnt(%1)\n\tds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v[0]) : "n"(W), "v"(a[0]));
  } else if constexpr (N == 2) {
    asm volatile("s_waitcnt vmcnt(%2)\n\tds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "n"(W), "v"(a[0]), "v"(a[1]));
  } else if constexpr (N == 3) {
    asm volatile("s_waitcnt vmcnt(%3)\n\tds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "n"(W), "v"(a[0]), "v"(a[1]), "v"(a[2]));
  } else {
    asm volatile("s_waitcnt vmcnt(%4)\n\tds_read_b128 %0, %5\n\tds_read_b128 %1, %6\n\tds_read_b128 %2, %7\n\t"
                 "ds_read_b128 %3, %8\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "n"(W), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
  }
}

// Next N chunks (N <= 4) with one LDS wait: vmcnt(kRing-N) means the N
// oldest DMAs (these slots) have landed, which holds only while all kRing
// slots have a DMA issued (owed == 0).  Then refill the N slots, or (refill
// false) leave them owed until ring_settle: no slot may be read while
// refills are owed, so only an instruction's last read defers them.
template <int N>
__device__ __forceinline__ void ring_read(Ring& r, u4 (&v)[4], bool refill = true) {
  static_assert(N >= 1 && N <= 4 && N <= kRing, "ring_read reads 1..4 chunks");
  uint32_t a[4];
  uint32_t slot = r.slot;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    a[k] = r.lds + slot * 1024 + lane_id() * 16;
    slot = (slot + 1 == kRing) ? 0 : slot + 1;
  }
  ring_load<N, kRing - N>(a, v);
  if (!refill) {
    r.slot = slot;
    r.owed += N;
    return;
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    dma_chunk(r.lds + r.slot * 1024, r.g, r.issue * 1024 + lane_id() * 16);
    r.issue = (r.issue + 1 == r.n) ? 0 : r.issue + 1;
    r.slot = (r.slot + 1 == kRing) ? 0 : r.slot + 1;
  }
}

// Issue the refills ring_read left owed, oldest slot first, so the ring's
// DMAs stay in slot order.
__device__ __forceinline__ void ring_settle(Ring& r) {
  uint32_t s = r.slot + kRing - r.owed;
  if (s >= (uint32_t)kRing) s -= kRing;
  for (uint32_t k = 0; k < r.owed; ++k) {
    dma_chunk(r.lds + s * 1024, r.g, r.issue * 1024 + lane_id() * 16);
    r.issue = (r.issue + 1 == r.n) ? 0 : r.issue + 1;
    s = (s + 1 == (uint32_t)kRing) ? 0 : s + 1;
  }
  r.owed = 0;
}


__device__ __forceinline__ float dot8(u4 w, const float* a) {
  const h8 h = __builtin_bit_cast(h8, w);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf((float)h[e], a[e], s);
  return s;
}


}  // namespace mk
