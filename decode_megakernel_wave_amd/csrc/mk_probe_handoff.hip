// mk_probe_handoff.hip -- calibration probe: latency of one cross-workgroup
// handoff (a system-scope store seen by a polling workgroup) while the chip
// streams weights through per-wavefront LDS rings the way the monokernel does
// (global_load_lds_dwordx4 ... nt, 12 x 1 KB slots per wavefront).
//
// Workgroup pairs ping-pong a counter: the leader stores r and polls for r
// from the follower, the follower polls for r and stores it back.  Half the
// round trip is one handoff.  What the other wavefronts do meanwhile is the
// variable:
//   mode 0  nothing streams;
//   mode 1  every CU streams on wavefronts 0-6, wavefront 7 of the pairs has
//           no ring and only polls;
//   mode 2  all 8 wavefronts of every CU stream, and the pairs' wavefront 7
//           consumes 4 chunks of its own ring before each handoff (its polls
//           and stores follow its refills, as in a GEMV instruction);
//   mode 3  the pairs' CUs stream nothing, every other CU streams on 8
//           wavefronts.
// Pairs are (2k, 2k+1) -- consecutive workgroups land on different XCDs -- or,
// with same_xcd, (k, k+8) in blocks of 16, which the round-robin dispatch puts
// on one XCD; the kernel records each member's XCC_ID so the host can report
// how many pairs really shared one.  Every wait is bounded by a spin limit.
//
// The file also holds the read-ceiling probe: the rate at which the chip
// streams a large buffer with nontemporal 16-byte loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"

namespace mk {
namespace {

constexpr int kProbeRing = 12;
constexpr int kProbePairs = 16;
constexpr int kProbeSpinLimit = 4000000;

struct HandoffArgs {
  const uint8_t* buf;    // stream source, n_chunks x 1 KB (< 4 GiB)
  uint32_t n_chunks;
  int32_t mode, same_xcd, rounds, stream_chunks;
  uint32_t* flags;       // [kProbePairs][2][64] words, zeroed
  uint64_t* ticks;       // [kProbePairs] device-clock ticks of the leader's `rounds` round trips
  int32_t* xcc;          // [kProbePairs][2] XCC_ID of leader and follower
  uint32_t* timeouts;    // waits that hit the spin limit
  u4* sink;              // [grid * 512] keeps the streamed data live
};

__device__ __forceinline__ u4 probe_slot_read(uint32_t a) {
  u4 v;
  asm volatile("s_waitcnt vmcnt(%1)\n\tds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "n"(kProbeRing - 1), "v"(a));
  return v;
}

extern __shared__ __attribute__((aligned(16))) uint8_t probe_smem[];

__global__ __launch_bounds__(512, 1) void mk_probe_handoff_k(HandoffArgs a) {
  const int wave = wave_id(), lane = lane_id(), wg = blockIdx.x;
  int pair = -1, leader = 0;
  if (a.same_xcd) {
    if (wg < 2 * kProbePairs) {
      const int blk = wg / 16, r = wg % 16;
      pair = blk * 8 + r % 8;
      leader = r < 8;
    }
  } else if (wg < 2 * kProbePairs) {
    pair = wg / 2;
    leader = wg % 2 == 0;
  }
  const bool streams = a.mode == 2 || (a.mode == 1 && wave < 7) || (a.mode == 3 && pair < 0);
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)probe_smem + wave * kProbeRing * 1024);
  uint32_t issue = ((uint32_t)(wg * 8 + wave) * 977u) % a.n_chunks;
  int slot = 0;
  u4 acc = {0u, 0u, 0u, 0u};
  auto consume = [&]() {
    acc ^= probe_slot_read(ring + slot * 1024 + lane * 16);
    dma_chunk(ring + slot * 1024, a.buf, issue * 1024 + lane * 16);
    issue = issue + 1 == a.n_chunks ? 0 : issue + 1;
    slot = slot + 1 == kProbeRing ? 0 : slot + 1;
  };
  if (streams) {
    for (int i = 0; i < kProbeRing; ++i) {
      dma_chunk(ring + i * 1024, a.buf, issue * 1024 + lane * 16);
      issue = issue + 1 == a.n_chunks ? 0 : issue + 1;
    }
  }
  if (wave == 7 && pair >= 0) {
    if (lane == 0) a.xcc[pair * 2 + (leader ? 0 : 1)] = xcc_id();
    // let the other wavefronts' streams ramp up (20 us)
    const uint64_t t_ramp = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t_ramp < 2000)
      if (streams) consume();
    uint32_t* mine = (uint32_t*)uniform_ptr(a.flags + (pair * 2 + (leader ? 0 : 1)) * 64);
    const uint32_t* other = (const uint32_t*)uniform_ptr(a.flags + (pair * 2 + (leader ? 1 : 0)) * 64);
    bool bad = false;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int r = 1; r <= a.rounds && !bad; ++r) {
      if (streams)
        for (int k = 0; k < 4; ++k) consume();
      if (leader && lane == 0) stc32(mine, (uint32_t)r);
      int spins = 0;
      while (__builtin_amdgcn_readfirstlane(ldc32(other)) != (uint32_t)r) {
        if (++spins > kProbeSpinLimit) {
          bad = true;
          break;
        }
      }
      if (!leader && lane == 0) stc32(mine, (uint32_t)r);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      if (bad) atomicAdd(a.timeouts, 1u);
      if (leader) a.ticks[pair] = t1 - t0;
    }
  } else if (streams) {
    for (int i = 0; i < a.stream_chunks; ++i) consume();
  }
  if (streams) {
    stores_acked();  // every DMA has landed before the workgroup's LDS goes away
    for (int i = 0; i < kProbeRing; ++i) {
      u4 v;
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(ring + i * 1024 + lane * 16));
      acc ^= v;
    }
  }
  a.sink[(int64_t)wg * 512 + threadIdx.x] = acc;
}

// Read ceiling: n16 16-byte words with nontemporal loads, in blocks of 16
// consecutive 1 KB chunks (one per load instruction of a wavefront, 16 KB in
// flight per wavefront), block b read by wavefront b mod (waves in the grid);
// then the chunks past the last whole block and the words past the last
// chunk.  The XOR of everything read goes to sink[thread] so that no load can
// be dropped.  (A grid-stride loop whose 8 loads per thread lay 8 MB apart
// read 6.0 TB/s; consecutive kilobytes per wavefront read 7.0.)
__global__ __launch_bounds__(512) void mk_probe_read_k(const u4* __restrict__ p, int64_t n16, u4* __restrict__ sink) {
  constexpr int kBlk = 16;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t nch = n16 / 64, nblk = nch / kBlk;
  u4 acc = {0u, 0u, 0u, 0u};
  for (int64_t b = wave; b < nblk; b += nwaves) {
    const u4* q = p + b * kBlk * 64 + lane;
    u4 v[kBlk];
#pragma unroll
    for (int k = 0; k < kBlk; ++k) v[k] = __builtin_nontemporal_load(q + k * 64);
#pragma unroll
    for (int k = 0; k < kBlk; ++k) acc ^= v[k];
  }
  for (int64_t c = nblk * kBlk + wave; c < nch; c += nwaves) acc ^= __builtin_nontemporal_load(p + c * 64 + lane);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (nch * 64 + t < n16) acc ^= __builtin_nontemporal_load(p + nch * 64 + t);
  sink[t] = acc;
}

}  // namespace
}  // namespace mk

#define MK_INTERNAL __attribute__((visibility("hidden")))

extern "C" {

// Launch over `grid` workgroups, one per CU (512 threads, 96 KB of LDS each).
MK_INTERNAL hipError_t mk_launch_probe_handoff(const void* buf, uint32_t n_chunks, int mode, int same_xcd, int rounds,
                                               int stream_chunks, uint32_t* flags, uint64_t* ticks, int32_t* xcc,
                                               uint32_t* timeouts, void* sink, int grid, hipStream_t s) {
  using namespace mk;
  const int lds = 8 * kProbeRing * 1024;
  hipError_t e = hipFuncSetAttribute((const void*)mk_probe_handoff_k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  HandoffArgs a{(const uint8_t*)buf, n_chunks, mode, same_xcd, rounds, stream_chunks, flags, ticks, xcc, timeouts, (u4*)sink};
  hipLaunchKernelGGL(mk_probe_handoff_k, dim3(grid), dim3(512), lds, s, a);
  return hipGetLastError();
}

MK_INTERNAL hipError_t mk_probe_handoff_occupancy(int* occupancy) {
  using namespace mk;
  const int lds = 8 * kProbeRing * 1024;
  hipError_t e = hipFuncSetAttribute((const void*)mk::mk_probe_handoff_k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, mk::mk_probe_handoff_k, 512, lds);
}

MK_INTERNAL int mk_probe_handoff_pairs() { return mk::kProbePairs; }

// The read-ceiling probe over `grid` workgroups of 512 threads; sink holds grid * 512 u4.
MK_INTERNAL hipError_t mk_launch_probe_read(const void* p, int64_t n16, void* sink, int grid, hipStream_t s) {
  hipLaunchKernelGGL(mk::mk_probe_read_k, dim3(grid), dim3(512), 0, s, (const mk::u4*)p, n16, (mk::u4*)sink);
  return hipGetLastError();
}

}  // extern "C"
