// mk_device.h -- gfx950 device primitives of the monokernel: coherent
// loads/stores for cross-workgroup sync, an LDS barrier for the compute
// wavefronts, wavefront DPP reductions, and the LDS weight rings that loader
// wavefronts fill with nontemporal global->LDS loads.
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

// Release / acquire between workgroups for data whose arrival the reader
// cannot see in the data itself (the KV cache and the sentinel re-arms at a
// step boundary; every stage in counter mode).  A system-scope store is
// acknowledged by the XCD's L2 before its write-through reaches memory, so
// waiting for the acknowledgements is not enough: the release also writes
// the L2 back (agent-scope release fence), and the acquire invalidates the
// reader's caches.  Measured: without the write-back, counter-mode consumers
// read values of the previous launch.
__device__ __forceinline__ void release_stores() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
// The wavefront's stores have reached the L2 (acknowledged).  A workgroup
// releases with: every wavefront waits for this, a barrier, then one
// wavefront's release fence writes the (shared) L2 back for all of them.
__device__ __forceinline__ void stores_acked() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void acquire_polled() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  uint64_t v = (uint64_t)p;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Barrier of the kWaves compute wavefronts, through an LDS counter.  The
// loader wavefronts never reach a barrier (they run their own loop), so the
// hardware s_barrier, which waits for every wavefront of the workgroup, is
// used only once, before the roles split.  Each wavefront adds 1 to the
// counter and waits until it reaches kWaves times the number of barriers it
// has entered (gen, a per-wavefront count kept by the caller).  The fences
// name the "local" address space only: global loads and stores in flight
// stay in flight across the barrier.
#define MK_LDS __attribute__((address_space(3)))
template <typename T>
__device__ __forceinline__ MK_LDS T* lp(T* p) { return (MK_LDS T*)p; }

// Returns false if the barrier did not complete within `ticks` of the device
// clock or the abort word became non-zero (the caller reports the fault).
__device__ __forceinline__ bool lds_barrier(uint32_t* bar, uint32_t& gen, uint64_t ticks, const uint32_t* abort) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  gen += kWaves;
  if (lane_id() == 0) __hip_atomic_fetch_add(lp(bar), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  uint32_t spins = 0;
  uint64_t deadline = 0;
  bool ok = true;
  while ((int32_t)(__hip_atomic_load(lp(bar), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) - gen) < 0) {
    if ((++spins & 255) == 0) {
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      if (deadline == 0) deadline = now + ticks;
      if (now > deadline || ldc32(abort) != 0) {
        ok = false;
        break;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return ok;
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

// ---------------------------------------------------------------- weight rings
// Each compute wavefront consumes one stream of 1 KB chunks (built by the
// host in consumption order, repeating every step) through a ring of kRing
// LDS slots.  A free slot holds the ring sentinel in every word.  A loader
// wavefront DMAs chunk i of the stream into slot i % kRing once the consumer
// has released the chunk that used the slot before (cons, the consumer's
// count of finished chunks, exceeds i - kRing).  The consumer reads a chunk
// until none of its words is the sentinel (the DMA has landed), then refills
// the slot with the sentinel and advances cons.  The loader therefore never
// waits for its DMAs to land; it only throttles how many are outstanding.
//
// The rings are touched only through inline asm (the DMA, the reads, the
// refills and the cons words), and volatile asm statements keep their
// program order, so none of them needs a "memory" clobber (which would make
// the compiler reload every value it keeps in memory after each chunk).

// Two fp16 NaNs with a full payload: no finite weight pair has this bit pattern.
constexpr uint32_t kRingSent = 0xFFFFFFFFu;

// LDS word access in program order with the ring asm (address = LDS byte offset).
__device__ __forceinline__ uint32_t lds_ld32(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ void lds_st32(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v));
}

// Loader side: DMA one chunk (64 lanes x 16 bytes) to LDS byte address
// lds_addr; lane i's bytes land at lds_addr + 16 i.  At most kInFlight DMAs
// of this wavefront stay outstanding (loads complete in order).
__device__ __forceinline__ void dma_chunk(uint32_t lds_addr, const uint8_t* g, uint32_t voff) {
  uint32_t save;
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  g = (const uint8_t*)uniform_ptr(g);
  asm volatile(
      "s_waitcnt vmcnt(%4)\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(voff), "s"(g), "n"(kInFlight - 1));
}

// Consumer side.
struct Ring {
  uint32_t lds;    // LDS byte address of this wavefront's ring
  uint32_t cons;   // LDS byte address of its consumed-count word
  uint32_t seq;    // chunks consumed so far in this launch
  uint32_t slot;   // seq % kRing
};

// Read the next N (1..4) chunks (16 bytes per lane each); true when every
// word of every lane has landed.
template <int N>
__device__ __forceinline__ bool ring_load(const Ring& r, u4 (&v)[4]) {
  static_assert(N >= 1 && N <= 4 && N <= kRing, "ring_load reads 1..4 chunks");
  uint32_t a[4];
  uint32_t slot = r.slot;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    a[k] = r.lds + slot * 1024 + lane_id() * 16;
    slot = (slot + 1 == kRing) ? 0 : slot + 1;
  }
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v[0]) : "v"(a[0]));
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(a[0]), "v"(a[1]));
  } else if constexpr (N == 3) {
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]));
  } else {
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
                 "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
  }
  bool pending = false;
#pragma unroll
  for (int k = 0; k < N; ++k)
    pending |= (v[k][0] == kRingSent) | (v[k][1] == kRingSent) | (v[k][2] == kRingSent) | (v[k][3] == kRingSent);
  return __ballot(pending) == 0;
}

// Release the N chunks just read: refill their slots with the sentinel, then
// advance cons (LDS executes a wavefront's accesses in order, so the loader
// never sees the new count before the refill).
template <int N>
__device__ __forceinline__ void ring_release(Ring& r) {
  const u4 s = {kRingSent, kRingSent, kRingSent, kRingSent};
#pragma unroll
  for (int k = 0; k < N; ++k) {
    asm volatile("ds_write_b128 %0, %1" ::"v"(r.lds + r.slot * 1024 + lane_id() * 16), "v"(s));
    r.slot = (r.slot + 1 == kRing) ? 0 : r.slot + 1;
  }
  r.seq += N;
  lds_st32(r.cons, r.seq);
}

__device__ __forceinline__ float dot8(u4 w, const float* a) {
  const h8 h = __builtin_bit_cast(h8, w);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf((float)h[e], a[e], s);
  return s;
}


}  // namespace mk
