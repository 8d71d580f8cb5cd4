// mk_kernel.hip -- the persistent decode monokernel for gfx950 (MI355X).
//
// One launch runs n decode steps.  Every workgroup (one per CU, sized by the
// occupancy query: "8 - Ecrire son megakernel", section 8.3) walks its own
// instruction list once per step ("8 - Ecrire son megakernel", section 8.2):
// fused RMSNorm+QKV+RoPE, split attention, the split merge, O-projection,
// gate/up, down projection, LM head and the greedy argmax.
//
// Synchronisation ("7 - AMD et le monokernel", section 7.3): every output
// buffer starts out holding a sentinel NaN bit pattern; producers overwrite
// it with agent-coherent stores and consumers poll each element they read
// with agent-coherent (L2-bypassing) loads until it is no longer the
// sentinel.  No counter, no fence per stage.  Each element is checked, which
// is the rule the page gives for writes that are not ordered among
// themselves.  Buffers rotate over three step epochs; the producer of an
// element re-arms it for the step after next.  One release fence per step
// (before the per-workgroup argmax key) orders the re-arms and KV writes.
// The atomic-counter protocol ("8 - Ecrire son megakernel", section 8.5:
// release fence, counter increment; acquire poll with back-off) is kept as
// a selectable comparison path on the same buffers.
//
// Weight streaming ("7 - AMD et le monokernel", section 7.5): each
// wavefront owns one contiguous stream of 1 KB chunks (built by the host in
// exactly the order the wavefront consumes them) and keeps kRing chunks in
// flight with nontemporal global->LDS loads, refilling a ring slot as soon as
// it has been read.  The ring runs across stage and step boundaries, so the
// next stage's weights are already arriving while the wavefront waits for
// its inputs.  GEMVs are fp16 x fp32 with fp32 accumulation and wavefront
// DPP reductions; no matrix cores are needed at batch 1.
//
// Per-XCD copies ("7 - AMD et le monokernel", section 7.4): vectors that
// every workgroup re-reads (residual stream, attention output, MLP
// activation, argmax keys) are written R times; a workgroup reads the copy
// of its own XCD.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mk_device.h"
#include "mk_layout.h"

// The file is compiled four times.  The general build holds mk_monokernel
// (every slice width, head_dim and sync mode) and the helper kernels.  With
// MK_SPECIALIZED it holds only one specialised interpreter, restricted to GEMV
// slices of four chunks (rows of 2048 or more columns), head_dim 128 with two
// query heads per kv head (the ~2B decoder's shapes) and one sync mode fixed
// at compile time (MK_SPEC_SYNC 0:
// sentinel, mk_monokernel_w4h128; 1: counter, mk_monokernel_w4h128_ctr).
// Leaving the other widths, head geometries and the other sync mode out of
// the kernel's code made the ~2B decode about 5 % faster (the interpreter's
// code is several times larger than the instruction cache); the host picks a
// specialised kernel when every instruction of the schedule fits it.  The
// fourth build (MK_LONG_DMA, sentinel sync, mk_monokernel_w4h128_long) streams
// long attention splits through LDS rings by DMA; the host runs it for
// launches whose splits are long from the first step (long contexts).  It is
// a kernel of its own because the monokernel is one function: inlined next to
// the short-context code, that pass changed the register allocation and code
// layout of the rest and made the 512-token decode 0.8 % slower.
#ifdef MK_SPECIALIZED
// query heads per kv head and head_dim the specialised build is compiled for
// (the host launches it only for that geometry); 0 = any
constexpr int kSpecGroup = 2;
constexpr int kSpecHd = 128;
#else
constexpr int kSpecGroup = 0;
constexpr int kSpecHd = 0;
#endif
#ifdef MK_SPECIALIZED
#if MK_SPEC_SYNC == 0 && defined(MK_LONG_DMA)
#define MK_MONOKERNEL mk_monokernel_w4h128_long
#define MK_SPEC_LAUNCH mk_launch_monokernel_w4h128_long
#define MK_SPEC_ATTR mk_kernel_attributes_w4h128_long
#elif MK_SPEC_SYNC == 0
#define MK_MONOKERNEL mk_monokernel_w4h128
#define MK_SPEC_LAUNCH mk_launch_monokernel_w4h128
#define MK_SPEC_ATTR mk_kernel_attributes_w4h128
#else
#define MK_MONOKERNEL mk_monokernel_w4h128_ctr
#define MK_SPEC_LAUNCH mk_launch_monokernel_w4h128_ctr
#define MK_SPEC_ATTR mk_kernel_attributes_w4h128_ctr
#endif
#else
#define MK_MONOKERNEL mk_monokernel
#endif

using namespace mk;

namespace {



// head_dim and query heads per kv head: compile-time constants in the specialised build
__device__ __forceinline__ int head_dim(const KParams& kp) { return kSpecHd ? kSpecHd : kp.hd; }
__device__ __forceinline__ int q_group(const KParams& kp) { return kSpecGroup ? kSpecGroup : kp.nq / kp.nkv; }

// ---------------------------------------------------------------- per-workgroup context
struct Smem {
  uint8_t* base;
  float* vec;        // staged input vector [kpad]
  float* scratch;    // [kScratchFloats]
  float* resid;      // [1024]
  uint32_t* flags;   // [2][kWaves] failure flags
  float* wsum;       // [kWaves] partial sums of squares
  uint64_t* keys;    // [kWaves]
  uint32_t* misc;    // [16]
};

struct Cx {
  const KParams* kp;
  Smem sm;
  int cta, wave, lane, tid, rep, xcc;
  int step, pos, e, e1, tok, pc;
  int flag_parity;
  bool fail;          // this thread saw a timeout or abort
  uint64_t deadline;
  int poll_iters;
};

__device__ __forceinline__ void raise_fault(Cx& c, int code, int op, int layer, int index) {
  const KParams& kp = *c.kp;
  MK_GLOBAL Fault* f = gp(kp.fault);
  int32_t expect = 0;
  if (__hip_atomic_compare_exchange_strong(&f->code, &expect, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    f->cta = c.cta;
    f->pc = c.pc;
    f->op = op;
    f->step = c.step;
    f->layer = layer;
    f->index = index;
  }
  if (code == -7) stc32(kp.abort_flag, 1u);
}

// Watchdog: called from poll loops; true when this thread must stop waiting.
__device__ __forceinline__ bool expired(Cx& c, int op, int layer, int index) {
  if ((++c.poll_iters & 63) != 0) return false;
  if (ldc32(c.kp->abort_flag)) return true;
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  if (c.deadline == 0) {
    c.deadline = now + c.kp->watchdog_ticks;
    return false;
  }
  if (now > c.deadline) {
    raise_fault(c, -7, op, layer, index);
    return true;
  }
  return false;
}

// Back-off between failed poll rounds: limits the coherent-load traffic that
// hundreds of waiting workgroups put on the memory system.
__device__ __forceinline__ void poll_pause(const Cx& c) {
  for (int i = 0; i < c.kp->poll_sleep; ++i) __builtin_amdgcn_s_sleep(1);
}

// One instruction record.  The lists do not change during a launch, so they
// are read through the constant address space: scalar loads into SGPRs.
__device__ __forceinline__ Ins load_ins(const Ins* p) {
  typedef const __attribute__((address_space(4))) u4 CU4;
  struct Raw {
    u4 a, b;
  } raw = {((CU4*)p)[0], ((CU4*)p)[1]};
  return __builtin_bit_cast(Ins, raw);
}

// Workgroup barrier.
__device__ __forceinline__ void cta_sync(Cx&) { cta_sync_hw(); }

// Workgroup-wide OR of the per-thread failure flags (also a barrier).
__device__ __forceinline__ bool cta_failed(Cx& c) {
  const uint64_t b = __ballot(c.fail);
  uint32_t* f = c.sm.flags + c.flag_parity * kWaves;
  if (c.lane == 0) f[c.wave] = b != 0;
  cta_sync(c);
  uint32_t any = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any |= f[w];
  c.flag_parity ^= 1;
  // the value is the same in every lane; say so, or every branch on it (and
  // the whole instruction loop) would be compiled as divergent
  return __builtin_amdgcn_readfirstlane(any) != 0;
}

// Diagnostics: fine timestamp k of the current instruction (step 0, thread 0).
// With MK_TSW the record instead holds, per wavefront w, the time its GEMV
// rows were done (slot w).
__device__ __forceinline__ void ts_mark(const Cx& c, int k) {
#ifndef MK_TSW
  if (c.kp->ts && c.step == 0 && c.tid == 0)
    *gp(c.kp->ts + ((int64_t)c.cta * c.kp->max_ins + c.pc) * 8 + k) = __builtin_amdgcn_s_memrealtime();
#endif
}

__device__ __forceinline__ void ts_wave_done(const Cx& c) {
#ifdef MK_TSW
  if (c.kp->ts && c.step == 0 && c.lane == 0)
    *gp(c.kp->ts + ((int64_t)c.cta * c.kp->max_ins + c.pc) * 8 + c.wave) = __builtin_amdgcn_s_memrealtime();
#endif
}

// Trace: time at which an instruction's inputs were staged.
__device__ __forceinline__ void mark_ready(Cx& c) {
  if (c.kp->trace && c.tid == 0 && c.step < c.kp->trace_steps) c.sm.misc[0] = (uint32_t)__builtin_amdgcn_s_memrealtime();
}

// Counter mode: one thread waits until the stage counter reaches its target.
#ifdef MK_SPECIALIZED
__device__ __forceinline__ bool sentinel_mode(const Cx&) { return MK_SPEC_SYNC == 0; }
#else
__device__ __forceinline__ bool sentinel_mode(const Cx& c) { return c.kp->sync_mode == 0; }
#endif

__device__ __forceinline__ void counter_wait(Cx& c, int sid, int n_in, int op, int layer) {
  if (sentinel_mode(c)) return;
  if (c.tid == 0 && sid >= 0) {
    const uint32_t target = (uint32_t)n_in * (uint32_t)(c.step + 1);
    uint32_t* ctr = c.kp->counters + sid;
    int tries = 0;
    while (!c.fail && __hip_atomic_load(gp(ctr), __ATOMIC_RELAXED, MK_SCOPE) < target) {
      // exponential back-off ("8 - Ecrire son megakernel", section 8.5)
      const int k = tries < 4 ? (1 << tries) : 16;
      for (int i = 0; i < k; ++i) __builtin_amdgcn_s_sleep(1);
      ++tries;
      if (expired(c, op, layer, sid)) {
        c.fail = true;
        break;
      }
    }
    acquire_polled();
  }
}

__device__ __forceinline__ void counter_signal(Cx& c, int sid) {
  if (sentinel_mode(c) || sid < 0) return;
  stores_acked();
  cta_sync(c);
  if (c.wave == 0) {
    release_stores();
    if (c.lane == 0) __hip_atomic_fetch_add(gp(c.kp->counters + sid), 1u, __ATOMIC_RELAXED, MK_SCOPE);
  }
}

// Poll one fp32 word until it stops being the sentinel (sentinel mode) or
// read it once (counter mode, after the counter wait).
__device__ __forceinline__ float poll_f32(Cx& c, const float* p, int op, int layer) {
  uint32_t v = ldc32(p);
  if (sentinel_mode(c)) {
    while (v == kSent32 && !c.fail) {
      if (expired(c, op, layer, -1)) {
        c.fail = true;
        break;
      }
      poll_pause(c);
      v = ldc32(p);
    }
  }
  return __uint_as_float(v);
}

__device__ __forceinline__ bool any_sent16(u4 v) {
  bool any = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) any |= (v[j] & 0xFFFFu) == kSent16 || (v[j] >> 16) == kSent16;
  return any;
}

__device__ __forceinline__ bool any_sent(u4 v) {
  return v[0] == kSent32 || v[1] == kSent32 || v[2] == kSent32 || v[3] == kSent32;
}

// Poll four consecutive fp32 sync words (16-byte aligned) until none is the
// sentinel (sentinel mode) or read them once (counter mode).
__device__ __forceinline__ u4 poll_f32x4(Cx& c, Rsrc rs, uint32_t byte_off, int op, int layer) {
  u4 v = ldc128(rs, byte_off);
  if (sentinel_mode(c)) {
    while (any_sent(v) && !c.fail) {
      if (expired(c, op, layer, -1)) {
        c.fail = true;
        break;
      }
      poll_pause(c);
      v = ldc128(rs, byte_off);
    }
  }
  return v;
}

// Stage n fp32 values of a sync buffer into LDS dst[0..npad) (zero padded),
// multiplied by the fp16 gain when one is given.  n is a multiple of 4 and src
// 16-byte aligned (every sync buffer is), so a thread reads 4 consecutive
// values per 16-byte request; all requests of a thread are issued before any
// is checked.  Returns this thread's sum of squares of the raw values (for
// RMSNorm).
__device__ __forceinline__ float stage_vec(Cx& c, const float* src, float* dst, int n, int npad, const uint16_t* gain, int op, int layer) {
  constexpr int kGroups = 4;  // 16-byte groups a thread stages per round
  const Rsrc rs = sync_rsrc(src, (uint32_t)n * 4u);
  float ss = 0.f;
  for (int base = c.tid * 4; base < npad; base += kThreads * 4 * kGroups) {
    u4 v[kGroups];
    float g[kGroups][4];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const int i = base + k * kThreads * 4;
      v[k] = i < n ? ldc128(rs, (uint32_t)i * 4u) : u4{0u, 0u, 0u, 0u};
      if (gain && i < n) {
        const u2 w = *gp((const u2*)(gain + i));
        const _Float16* h = (const _Float16*)&w;
#pragma unroll
        for (int j = 0; j < 4; ++j) g[k][j] = (float)h[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) g[k][j] = 1.f;
      }
    }
    if (sentinel_mode(c)) {
      // re-poll every group still holding a sentinel in one batch, so a late
      // producer costs one more round trip, not one per element
      for (;;) {
        bool pending = false;
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
          const int i = base + k * kThreads * 4;
          pending |= i < n && any_sent(v[k]);
        }
        if (!pending || c.fail) break;
        if (expired(c, op, layer, base)) {
          c.fail = true;
          break;
        }
        poll_pause(c);
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
          const int i = base + k * kThreads * 4;
          if (i < n && any_sent(v[k])) v[k] = ldc128(rs, (uint32_t)i * 4u);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const int i = base + k * kThreads * 4;
      if (i < npad) {
        f4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float f = __uint_as_float(v[k][j]);
          ss += f * f;
          x[j] = f * g[k][j];
        }
        *(f4*)(dst + i) = x;
      }
    }
  }
  return ss;
}

// Stage an fp16 row of read-only data (an embedding row) as fp32, times the
// gain; returns this thread's sum of squares of the raw values.
__device__ __forceinline__ float stage_row_h(Cx& c, const uint16_t* src, float* dst, int n, int npad, const uint16_t* gain) {
  float ss = 0.f;
  for (int i = c.tid * 4; i < npad; i += kThreads * 4) {
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (i < n) {
      const u2 w = *gp((const u2*)(src + i));
      const u2 gw = *gp((const u2*)(gain + i));
      const _Float16* h = (const _Float16*)&w;
      const _Float16* gh = (const _Float16*)&gw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float f = (float)h[j];
        ss += f * f;
        v[j] = f * (float)gh[j];
      }
    }
    *(f4*)(dst + i) = v;
  }
  return ss;
}

__device__ __forceinline__ float* buf_at(const Buf& b, int e, int l, int r) {
  return b.p + e * b.es + (int64_t)l * b.ls + (int64_t)r * b.rs;
}

// Store value v at element idx of every replica of b (epoch e) and re-arm the
// same element for epoch e1 (sentinel mode).  Called by the whole wavefront
// with a uniform value; lanes 0..R-1 store, lanes R..2R-1 re-arm.
__device__ __forceinline__ void publish(const Cx& c, const Buf& b, int l, int64_t idx, float v) {
  const int R = c.kp->R;
  if (c.lane < R) stcf(buf_at(b, c.e, l, c.lane) + idx, v);
  else if (c.lane < 2 * R && sentinel_mode(c)) stc32(buf_at(b, c.e1, l, c.lane - R) + idx, kSent32);
}

// Rows [u0, u0 + nu) of b (epoch e) from LDS src to every replica, with
// stores that are contiguous across the lanes of a wavefront, then (when
// `rearm`) the same rows of epoch e1 back to the sentinel.  A GEMV that owns
// a contiguous range of output rows writes them this way after its last row,
// so the memory system sees a few full-line writes per replica instead of
// one partial-line write per element and replica.
__device__ __forceinline__ void publish_rows(const Cx& c, const Buf& b, int e, int l, int u0, int nu, const float* src, bool rearm) {
  const int R = c.kp->R, n = nu * R;
  for (int i = c.tid; i < n; i += kThreads) {
    const int r = i / nu, k = i - r * nu;
    stcf(buf_at(b, e, l, r) + u0 + k, src[k]);
  }
  if (rearm && sentinel_mode(c)) {
    for (int i = c.tid; i < n; i += kThreads) {
      const int r = i / nu, k = i - r * nu;
      stc32(buf_at(b, c.e1, l, r) + u0 + k, kSent32);
    }
  }
}

// Output rows a GEMV instruction can stage in LDS (sm.resid) before
// publish_rows; longer ranges (very small grids) publish row by row.
__device__ __forceinline__ bool staged_rows(const Ins& in) {
#ifdef MK_DIRECT_PUBLISH
  return false;
#else
  return in.nu <= kResidRows;
#endif
}

// ---------------------------------------------------------------- GEMV core
// The next n (1..4, uniform) chunks of the ring.
__device__ __forceinline__ void ring_read_n(Ring& ring, u4 (&w)[4], int n, bool refill) {
  switch (n) {
    case 4: ring_read<4>(ring, w, refill); break;
    case 3: ring_read<3>(ring, w, refill); break;
    case 2: ring_read<2>(ring, w, refill); break;
    default: ring_read<1>(ring, w, refill); break;
  }
}

// The refills of a wavefront's last ring read in an instruction (the second
// read of a two-row unit) are left owed until the instruction's outputs are
// published (ring_settle at the end of the op).  A CU's sync stores and loads
// wait behind the weight requests that CU has in flight: a handoff between two
// CUs that stream takes about 1.8 us, between two that do not 0.6-0.8 us, with
// the rest of the chip streaming in both cases.  Issuing the last refills after
// the stores lets the outputs leave first.  QKV's are issued later still, in
// the attention stage after its q polls, K/V loads and the split's published
// partials (the attention reads no weights, so they still land before the
// next GEMV): 2 % faster
// decode than issuing them after QKV's stores, where they sat ahead of those
// polls.  The
// other GEMVs' could not wait that long: issued only after the next GEMV had
// staged its inputs, they arrived late for it (4 % slower).

// GEMV body.  CPS = 4: slices of four chunks, the widest and the common case
// (rows of 2048 or more columns); CPS = 0: any width in.cps = 1..4 with
// uniform guards on the chunk loops.  Two bodies per op instead of one per
// width: the monokernel's code is far larger than the instruction cache.
template <int CPS, typename Epi>
__device__ __forceinline__ void gemv(Cx& c, Ring& ring, const Ins& in, const float* vec, float scale, Epi epi) {
  ring_settle(ring);  // refills an earlier instruction left owed (none unless it deferred them)
  const int ks = in.ks, rg = kWaves / ks, ki = c.wave % ks, gi = c.wave / ks;
  const int upr = in.upr, cps = CPS ? CPS : in.cps;
  float act[4][8];
  const int col0 = ki * cps * kChunkHalfs + c.lane * 8;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (CPS || k < cps) {
      a = *(const f4*)(vec + col0 + k * kChunkHalfs);
      b = *(const f4*)(vec + col0 + k * kChunkHalfs + 4);
    }
    act[k][0] = a[0]; act[k][1] = a[1]; act[k][2] = a[2]; act[k][3] = a[3];
    act[k][4] = b[0]; act[k][5] = b[1]; act[k][6] = b[2]; act[k][7] = b[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) act[k][e] *= scale;
  }
  ts_mark(c, 5);
  for (int u = gi; u < in.nu; u += rg) {
    float r0 = 0.f, r1 = 0.f;
    u4 w[4];
    const bool refill = u + rg < in.nu;  // false: this wavefront's last unit
    const bool refill0 = refill || upr == 2;
    if constexpr (CPS > 0) ring_read<CPS>(ring, w, refill0);
    else ring_read_n(ring, w, cps, refill0);
    if (u == gi) ts_mark(c, 7);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (CPS ? k < CPS : k < cps) r0 += dot8(w[k], act[k]);
    if (upr == 2) {
      if constexpr (CPS > 0) ring_read<CPS>(ring, w, refill);
      else ring_read_n(ring, w, cps, refill);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (CPS ? k < CPS : k < cps) r1 += dot8(w[k], act[k]);
    }
    r0 = wave_sum(r0);
    if (upr == 2) r1 = wave_sum(r1);
    if (ks == 1) {
      epi(u, r0, r1);
    } else if (c.lane == 0) {
      c.sm.scratch[(u * upr) * ks + ki] = r0;
      if (upr == 2) c.sm.scratch[(u * upr + 1) * ks + ki] = r1;
    }
  }
  ts_mark(c, 6);
  ts_wave_done(c);
  if (ks > 1) {
    cta_sync(c);
    if (ki == 0) {
      // one unit per lane: sum its ks partials (fixed order), then hand each
      // sum to the epilogue as a uniform value
      const int mine = units_of_group(in.nu, rg, gi);
      for (int base = 0; base < mine; base += 64) {
        const int j = base + c.lane;
        float s0 = 0.f, s1 = 0.f;
        if (j < mine) {
          const int u = gi + j * rg;
          for (int k = 0; k < ks; ++k) s0 += c.sm.scratch[(u * upr) * ks + k];
          if (upr == 2)
            for (int k = 0; k < ks; ++k) s1 += c.sm.scratch[(u * upr + 1) * ks + k];
        }
        const int cnt = min(64, mine - base);
        for (int t = 0; t < cnt; ++t) {
          const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s0), t));
          const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s1), t));
          epi(gi + (base + t) * rg, a, b);
        }
      }
    }
  }
}

template <typename Epi>
__device__ __forceinline__ void gemv_dispatch(Cx& c, Ring& ring, const Ins& in, const float* vec, float scale, Epi epi) {
#ifdef MK_SPECIALIZED
  gemv<4>(c, ring, in, vec, scale, epi);
#else
  if (in.cps == 4) gemv<4>(c, ring, in, vec, scale, epi);
  else gemv<0>(c, ring, in, vec, scale, epi);
#endif
}

// Closes the staging of an instruction's inputs: barrier, trace mark and,
// for RMSNorm inputs, the workgroup sum of squares of the n staged values
// (ss_thread = this thread's share).  Returns the RMSNorm scale (1 without norm).
__device__ __forceinline__ float finish_staging(Cx& c, int n, bool norm, float ss_thread) {
  ts_mark(c, 1);
  if (norm) {
    const float p = wave_sum(ss_thread);
    if (c.lane == 0) c.sm.wsum[c.wave] = p;
  }
  cta_sync(c);
  ts_mark(c, 2);
  mark_ready(c);
  if (!norm) return 1.0f;
  float ss = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ss += c.sm.wsum[w];
  return 1.0f / __builtin_sqrtf(ss / (float)n + c.kp->eps);
}

// Stage the layer input x_l (embedding row for layer 0) times the gain.
__device__ __forceinline__ float stage_layer_input(Cx& c, int l, int npad, const uint16_t* gain, int op) {
  const KParams& kp = *c.kp;
  if (l == 0) return stage_row_h(c, kp.embed + (int64_t)c.tok * kp.d, c.sm.vec, kp.d, npad, gain);
  return stage_vec(c, buf_at(kp.xm, c.e, l - 1, c.rep), c.sm.vec, kp.d, npad, gain, op, l);
}

// Residual rows [u0, u0+nu) of x_l (embedding for layer 0) into sm.resid, in
// two halves around the staging of the instruction's main input: the rows
// were published a stage or more earlier, so resid_issue loads this thread's
// first row before the main input is polled (its value is then back when the
// polls are), and resid_finish stores it, re-polling only if it was still
// the sentinel, plus any rows beyond the first kThreads.
__device__ __forceinline__ uint32_t resid_issue(Cx& c, const float* src, const uint16_t* emb, int u0, int nu) {
  if (c.tid >= nu) return 0u;
  if (emb) return (uint32_t)*gp(emb + u0 + c.tid);
  return ldc32(src + u0 + c.tid);
}

__device__ __forceinline__ void resid_finish(Cx& c, uint32_t first, const float* src, const uint16_t* emb, int u0, int nu, int op,
                                             int layer) {
  for (int i = c.tid; i < nu; i += kThreads) {
    float v;
    if (emb) {
      v = (float)__builtin_bit_cast(_Float16, (uint16_t)(i == c.tid ? first : (uint32_t)*gp(emb + u0 + i)));
    } else if (i == c.tid && (!sentinel_mode(c) || first != kSent32)) {
      v = __uint_as_float(first);
    } else {
      v = poll_f32(c, src + u0 + i, op, layer);
    }
    c.sm.resid[i] = v;
  }
}

// ---------------------------------------------------------------- ops
__device__ __forceinline__ void op_qkv(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int l = in.layer;
  counter_wait(c, in.sync_in, in.n_in, OP_QKV, l);
  if (!sentinel_mode(c)) cta_sync(c);
  const uint16_t* g1 = kp.norms + (int64_t)l * 2 * kp.d;
  // the (cos, sin) row of this position goes to LDS with the staging, so the
  // epilogue does not wait on a global load per unit
  const int hh = head_dim(kp) / 2, nqh = kp.nq * hh, nkh = kp.nkv * hh;
  float* rope = c.sm.resid;
  // loaded before the input is polled but stored to LDS after it: a wait for this load right away
  // would also wait for every weight DMA in flight before the polls are even issued
  static_assert(kThreads >= 2 * 128, "one RoPE value per thread (head_dim <= 256)");
  const float rv = c.tid < 2 * hh ? *gp(kp.rope + (int64_t)c.pos * hh * 2 + c.tid) : 0.f;
  const float ss = stage_layer_input(c, l, in.kpad, g1, OP_QKV);
  if (c.tid < 2 * hh) rope[c.tid] = rv;
  const float scale = finish_staging(c, kp.d, true, ss);
  // Output element `half` (0: row i, 1: row i + hd/2) of global unit g: a
  // rotary pair of a q head (fp32, one copy, the other epoch re-armed) or a
  // k head (fp16 into the cache) after RoPE, or a pair of value rows.
  auto store_out = [&](int g, int half, float v) {
    if (g < nqh) {
      const int64_t idx = (int64_t)(g / hh) * head_dim(kp) + g % hh + half * hh;
      stcf(buf_at(kp.q, c.e, l, 0) + idx, v);
      if (sentinel_mode(c)) stc32(buf_at(kp.q, c.e1, l, 0) + idx, kSent32);
    } else {
      const bool isk = g < nqh + nkh;
      g -= isk ? nqh : nqh + nkh;
      const int64_t idx = (((int64_t)l * kp.nkv + g / hh) * kp.max_seq + c.pos) * head_dim(kp) + g % hh + half * hh;
      stc16((isk ? kp.kc : kp.vc) + idx, __builtin_bit_cast(uint16_t, (_Float16)v));
    }
  };
  // outputs are staged after the RoPE row and written together at the end
  float* outs = rope + 2 * hh;  // [2][nu]
  const bool staged = staged_rows(in) && 2 * hh + 2 * in.nu <= kResidRows;
  gemv_dispatch(c, ring, in, c.sm.vec, scale, [&](int u, float a, float b) {
    const int g = in.u0 + u;
    if (g < nqh + nkh) {  // rotary pair (i, i + hd/2) of a q or k head
      const int i = (g < nqh ? g : g - nqh) % hh;
      const float cs = rope[2 * i], sn = rope[2 * i + 1];
      const float ra = a * cs - b * sn, rb = a * sn + b * cs;
      a = ra;
      b = rb;
    }
    if (staged) {
      if (c.lane == 0) {
        outs[u] = a;
        outs[in.nu + u] = b;
      }
    } else if (c.lane < 2) {
      store_out(g, c.lane, c.lane == 0 ? a : b);
    }
  });
  if (staged) {
    cta_sync(c);
    for (int t = c.tid; t < 2 * in.nu; t += kThreads) store_out(in.u0 + t % in.nu, t / in.nu, outs[t]);
  }
  // the refills left owed go out in the attention stage, after its q polls and K/V loads (a workgroup
  // without attention units issues them at its next GEMV)
  counter_signal(c, in.sync_out);
}

// Merge the S splits of query head h for output dims [b * kRedDims, +kRedDims):
// one wavefront, lane s holds split s; publishes o (every replica).
static_assert(kRedDims * 8 <= 64, "red_unit stores kRedDims dims to up to 8 replicas from one wavefront");
__device__ __forceinline__ void red_unit(Cx& c, int l, int h, int b) {
  const KParams& kp = *c.kp;
  const int hd = head_dim(kp), S = kp.S;
  const int s = c.lane;
  const int64_t base = (((int64_t)c.e * kp.L + l) * kp.nq + h) * S + s;
  float ms = -INFINITY, ls = 0.f, os[kRedDims];
#pragma unroll
  for (int d = 0; d < kRedDims; ++d) os[d] = 0.f;
  if (s < S) {
    // (m, l) is 8-byte aligned, the kRedDims output dims 32-byte aligned:
    // one 8-byte and two 16-byte system-scope loads per split, re-issued
    // together while any word is still the sentinel
    static_assert(kRedDims == 8, "red_unit loads its dims as two 16-byte groups");
    // the resources start at split 0 (uniform); lane s reads at its own offset
    const int64_t base0 = base - s;
    const Rsrc rml = sync_rsrc(kp.att_ml + base0 * 2, (uint32_t)S * 8u);
    const Rsrc rov = sync_rsrc(kp.att_o + base0 * hd, (uint32_t)(S * hd) * 4u);
    const uint32_t oml = (uint32_t)s * 8u, oov = (uint32_t)(s * hd + b * kRedDims) * 4u;
    u2 ml = ldc64v(rml, oml);
    u4 o0 = ldc128(rov, oov), o1 = ldc128(rov, oov + 16u);
    if (sentinel_mode(c)) {
      while ((ml[0] == kSent32 || ml[1] == kSent32 || any_sent(o0) || any_sent(o1)) && !c.fail) {
        if (expired(c, OP_ATT, l, h)) {
          c.fail = true;
          break;
        }
        poll_pause(c);
        ml = ldc64v(rml, oml);
        o0 = ldc128(rov, oov);
        o1 = ldc128(rov, oov + 16u);
      }
    }
    ms = __uint_as_float(ml[0]);
    ls = __uint_as_float(ml[1]);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      os[d] = __uint_as_float(o0[d]);
      os[4 + d] = __uint_as_float(o1[d]);
    }
  }
  const float M = wave_max(ms);
  const float w = (s < S && ms != -INFINITY) ? exp2f(ms - M) : 0.f;
  const float Lt = wave_sum(w * ls);
  const float inv = 1.0f / Lt;
  // lane r * kRedDims + d stores dim d to replica r: one contiguous
  // kRedDims-float write per replica (and one re-arm write per replica)
  const int rr = c.lane / kRedDims, dl = c.lane % kRedDims;
  float mine = 0.f;
#pragma unroll
  for (int d = 0; d < kRedDims; ++d) {
    const float v = wave_sum(w * os[d]) * inv;
    if (dl == d) mine = v;
  }
  if (rr < kp.R) {
    const int64_t idx = (int64_t)h * hd + b * kRedDims + dl;
    stcf(buf_at(kp.o, c.e, l, rr) + idx, mine);
    if (sentinel_mode(c)) stc32(buf_at(kp.o, c.e1, l, rr) + idx, kSent32);
  }
}

// Split attention for (kv head, split) units: unnormalised partial
// O = sum_t 2^(s_t - m) v_t, L = sum_t 2^(s_t - m), m = max_t s_t, with
// scores s_t = q.k_t / sqrt(hd) * log2(e).
//
// Query heads [j0, j0 + ng) of the group (ng <= GP) over the positions
// [t0, t1), for head_dim HD.  A K or V row is HD fp16 = HD / 8 lanes of 16
// bytes, so one 16-byte load per lane covers PPI = 512 / HD positions: lane
// `lane` holds dims [dl * 8, dl * 8 + 8) of position slot `sub`.  Each
// wavefront takes position groups wave, wave + kWaves, ... and keeps up to
// 8 groups of K and V loads in flight before computing; every lane
// keeps its own online-softmax state (m, l, o) for its slot, the slots are
// merged with cross-lane shuffles, then the wavefronts through the scratch.

// Short splits (at most kPosBatch positions per wavefront): query heads
// [j0, j0 + ng) of the group (ng <= GP) over the positions [t0, t1); wavefront
// w holds positions t0 + w + b * kWaves (b < kPosBatch) in kv / vv, lane i
// dims [i*DPL, i*DPL + DPL).  GP * DPL <= 8 keeps the accumulators in 8
// registers per lane whatever the head geometry.

template <int GP, int DPL>
__device__ __forceinline__ void att_pos_core(Cx& c, Ring& ring, int l, int g, int sp, int j0, int ng, int t0, int t1, int G,
                                             const float (&kv)[kPosBatch][DPL], const float (&vv)[kPosBatch][DPL]) {
  const KParams& kp = *c.kp;
  const int hd = head_dim(kp), S = kp.S;
  const float* qs = c.sm.vec;  // [G][hd]
  float m[GP], lsum[GP], o[GP][DPL];
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[j][k] = 0.f;
  }
  {
    // The wavefront's nb positions tb, tb + kWaves, ... (nb <= kPosBatch,
    // uniform) are one batch: every score first -- the wavefront sums do not
    // depend on each other, so they overlap -- then per head the batch maximum,
    // the weights 2^(s - m), their sum and the weighted V sum.  Positions past
    // nb hold zero K/V rows; their sums are computed and ignored.
    const int tb = t0 + c.wave;
    const int nb = tb < t1 ? min(kPosBatch, (t1 - tb + kWaves - 1) / kWaves) : 0;
    float sc[GP][kPosBatch];
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      if (GP != kSpecGroup && j >= ng) break;
      float qv[DPL];
#pragma unroll
      for (int k = 0; k < DPL; ++k) qv[k] = qs[(j0 + j) * hd + c.lane * DPL + k];
#pragma unroll
      for (int b = 0; b < kPosBatch; ++b) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) s += qv[k] * kv[b][k];
        sc[j][b] = s;
      }
    }
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      if (GP != kSpecGroup && j >= ng) break;
#pragma unroll
      for (int b = 0; b < kPosBatch; ++b) sc[j][b] = wave_sum(sc[j][b]);
    }
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      if (GP != kSpecGroup && j >= ng) break;
      float mn = -INFINITY;
#pragma unroll
      for (int b = 0; b < kPosBatch; ++b)
        if (b < nb) mn = fmaxf(mn, sc[j][b]);
#pragma unroll
      for (int b = 0; b < kPosBatch; ++b) {
        if (b < nb) {
          const float p = exp2f(sc[j][b] - mn);
          lsum[j] += p;
#pragma unroll
          for (int k = 0; k < DPL; ++k) o[j][k] += p * vv[b][k];
        }
      }
      m[j] = mn;
    }
  }
  ts_mark(c, 5);
  // combine the wavefronts: scratch [wave][ng][hd + 2]
  float* scr = c.sm.scratch;
  const int rec = hd + 2;
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    if (GP != kSpecGroup && j >= ng) break;
    float* r = scr + (c.wave * ng + j) * rec;
#pragma unroll
    for (int k = 0; k < DPL; ++k) r[2 + c.lane * DPL + k] = o[j][k];
    if (c.lane == 0) {
      r[0] = m[j];
      r[1] = lsum[j];
    }
  }
  cta_sync(c);
  ts_mark(c, 7);
  for (int i = c.tid; i < ng * hd; i += kThreads) {
    const int j = i / hd, dd = i % hd;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, scr[(w * ng + j) * rec]);
    float Lt = 0.f, Ot = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float* r = scr + (w * ng + j) * rec;
        const float al = exp2f(r[0] - M);
        Lt += al * r[1];
        Ot += al * r[2 + dd];
      }
    }
    const int qh = g * G + j0 + j;
    const int64_t po = ((((int64_t)c.e * kp.L + l) * kp.nq + qh) * S + sp);
    const int64_t po1 = ((((int64_t)c.e1 * kp.L + l) * kp.nq + qh) * S + sp);
    stcf(kp.att_o + po * hd + dd, Ot);
    if (sentinel_mode(c)) stc32(kp.att_o + po1 * hd + dd, kSent32);
    if (dd == 0) {
      stcf(kp.att_ml + po * 2, M);
      stcf(kp.att_ml + po * 2 + 1, Lt);
      if (sentinel_mode(c)) {
        stc32(kp.att_ml + po1 * 2, kSent32);
        stc32(kp.att_ml + po1 * 2 + 1, kSent32);
      }
    }
  }
  // the refills QKV left owed go out here, behind the q polls, the K/V loads and the split's
  // published partials, which would otherwise leave the CU behind them: 447.9 vs 451.5 ms per 512
  // tokens against issuing them before the wavefronts combine (456.3 there vs 457.3 before the
  // scores, where they could hold the wavefront at the issue); issued only after the split merge
  // they arrive late for O-proj (464.1 vs 449.8)
  ring_settle(ring);
  cta_sync(c);  // scratch reused by the next pass
}

// Sum over each aligned group of LPP lanes (8, 16 or 32), in every lane of
// the group: DPP within 16-lane rows, one permute across rows for 32.
template <int LPP>
__device__ __forceinline__ float slot_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror: 8-lane sums
  if constexpr (LPP >= 16) v += dpp<0x140>(v);  // row_mirror: 16-lane sums
  if constexpr (LPP >= 32) v += __shfl_xor(v, 16);
  return v;
}

#ifdef MK_LONG_DMA
// A long split's K/V ring of one wavefront: two slots of one position group
// (PPI = 512 / HD consecutive rows: 1 KB of K, then 1 KB of V), filled by DMA
// (global -> LDS, nontemporal), in the staged vector after q and the current
// K/V row (the plan sizes the vector for it).  The wavefront's groups are
// wave, wave + kWaves, ...: `mine` of them.
struct KvRing {
  uint32_t ring0;
  const uint8_t* kg;
  const uint8_t* vg;
  int mine;
};

template <int HD>
__device__ __forceinline__ KvRing kv_ring(const Cx& c, int l, int g, int t0, int t1, int G) {
  constexpr int PPI = 512 / HD;
  const KParams& kp = *c.kp;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // the kernel's dynamic LDS
  const int ngroups = (t1 - t0 + PPI - 1) / PPI;
  const int64_t head_row0 = ((int64_t)l * kp.nkv + g) * kp.max_seq;
  KvRing r;
  r.ring0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + (uint32_t)((const uint8_t*)c.sm.vec - c.sm.base) +
                                          (uint32_t)(att_ring_offset(G, HD) * 4 + c.wave * 4096));
  r.kg = (const uint8_t*)uniform_ptr(kp.kc + head_row0 * HD);
  r.vg = (const uint8_t*)uniform_ptr(kp.vc + head_row0 * HD);
  r.mine = ngroups > c.wave ? (ngroups - c.wave + kWaves - 1) / kWaves : 0;
  return r;
}

// DMA of the wavefront's group i (< r.mine) into slot i % 2; lanes past the
// split read the split's last row (valid, unused).
template <int HD>
__device__ __forceinline__ void kv_issue(const Cx& c, const KvRing& r, int t0, int t1, int i) {
  constexpr int LPP = HD / 8, PPI = 64 / LPP;
  const int sub = c.lane / LPP, dl = c.lane % LPP;
  const int t = min(t0 + (c.wave + i * kWaves) * PPI + sub, t1 - 1);
  const uint32_t voff = (uint32_t)t * (uint32_t)(HD * 2) + (uint32_t)dl * 16u;
  const uint32_t slot = r.ring0 + (uint32_t)(i & 1) * 2048u;
  dma_chunk(slot, r.kg, voff);
  dma_chunk(slot + 1024u, r.vg, voff);
}
#endif

template <int HD, int GP>
__device__ __forceinline__ void att_pass(Cx& c, int l, int g, int sp, int j0, int ng, int t0, int t1, int G, int pre = 0) {
  const KParams& kp = *c.kp;
  const int S = kp.S;
  constexpr int LPP = HD / 8, PPI = 64 / LPP;
  const int sub = c.lane / LPP, dl = c.lane % LPP;
  const float* qs = c.sm.vec;            // [G][HD]
  const float* kcur = c.sm.vec + G * HD; // [HD]
  const float* vcur = kcur + HD;         // [HD]
  float q[GP][8], m[GP], lsum[GP], o[GP][8];
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[j][e] = 0.f;
      q[j][e] = j < ng ? qs[(j0 + j) * HD + dl * 8 + e] : 0.f;
    }
  }
#ifdef MK_LONG_DMA
  // one position group (PPI positions, one per lane slot) into the online softmax, rounded as the
  // register path rounds: rows past the split and the current position's row (read from LDS
  // instead) are zeroed as raw bits first, and the two updates are written as the fused forms
  // the compiler chooses there, so this kernel's logits are bitwise those of the others
  auto group = [&](int grp, u4 kq, u4 vq) {
    const int t = t0 + grp * PPI + sub;
    const bool valid = t < t1;
    if (!valid || t == c.pos) {
      kq = u4{0u, 0u, 0u, 0u};
      vq = u4{0u, 0u, 0u, 0u};
    }
    float kf[8], vf[8];
    const h8 kh = __builtin_bit_cast(h8, kq), vh = __builtin_bit_cast(h8, vq);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = t == c.pos ? kcur[dl * 8 + e] : (float)kh[e];
      vf[e] = t == c.pos ? vcur[dl * 8 + e] : (float)vh[e];
    }
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      if (GP != kSpecGroup && j >= ng) break;
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc = fmaf(q[j][e], kf[e], sc);
      sc = slot_sum<LPP>(sc);
      const float mn = valid ? fmaxf(m[j], sc) : m[j];
      const float al = mn == -INFINITY ? 0.f : exp2f(m[j] - mn);
      const float pv = valid ? exp2f(sc - mn) : 0.f;
      lsum[j] = fmaf(lsum[j], al, pv);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = fmaf(vf[e], pv, o[j][e] * al);
      m[j] = mn;
    }
  };
  // K/V through the wavefront's 2-group LDS ring, a slot's refill issued as soon as the slot is
  // read.  With every workgroup starting its split at once, the CU streams these faster than the
  // same bytes loaded into registers (probe of an 8192-token context: 12.1 vs 14.0 us per layer
  // with 8 groups per wavefront in registers).  `pre` groups were issued before q was polled.
  const KvRing r = kv_ring<HD>(c, l, g, t0, t1, G);
  const int mine = r.mine;
  for (int i = pre; i < 2 && i < mine; ++i) kv_issue<HD>(c, r, t0, t1, i);
  for (int i = 0; i < mine; ++i) {
    const uint32_t a = r.ring0 + (uint32_t)(i & 1) * 2048u + (uint32_t)c.lane * 16u;
    u4 kq, vq;
    // this group's two DMAs have landed when at most the next group's two are outstanding
    if (i + 1 < mine)
      asm volatile("s_waitcnt vmcnt(2)\n\tds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(kq), "=&v"(vq) : "v"(a));
    else
      asm volatile("s_waitcnt vmcnt(0)\n\tds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(kq), "=&v"(vq) : "v"(a));
    if (i + 2 < mine) kv_issue<HD>(c, r, t0, t1, i + 2);
    if (i == 0) ts_mark(c, 5);  // the first group landed
    group(c.wave + i * kWaves, kq, vq);
  }
#else
  constexpr int kAttBatch = GP >= 4 ? 4 : 8;  // position groups in flight (registers: 8 per group)
  const int64_t head_off = ((int64_t)l * kp.nkv + g) * kp.max_seq * HD + dl * 8;
  const uint16_t* kbase = kp.kc + head_off;
  const uint16_t* vbase = kp.vc + head_off;
  const int ngroups = (t1 - t0 + PPI - 1) / PPI;
  for (int gb = c.wave; gb < ngroups; gb += kWaves * kAttBatch) {
    u4 kb[kAttBatch], vb[kAttBatch];
#pragma unroll
    for (int b = 0; b < kAttBatch; ++b) {
      const int t = t0 + (gb + b * kWaves) * PPI + sub;
      if (t < t1 && t != c.pos) {
        // read once per token: nontemporal, like the weights (286 vs 292 ms per 256 tokens at an
        // 8192-token context against loads with the default cache policy)
        kb[b] = __builtin_nontemporal_load(gp((const u4*)(kbase + (int64_t)t * HD)));
        vb[b] = __builtin_nontemporal_load(gp((const u4*)(vbase + (int64_t)t * HD)));
      } else {
        kb[b] = u4{0u, 0u, 0u, 0u};
        vb[b] = u4{0u, 0u, 0u, 0u};
      }
    }
    if (gb == c.wave) ts_mark(c, 5);  // the first batch of K/V loads issued
#pragma unroll
    for (int b = 0; b < kAttBatch; ++b) {
      const int t = t0 + (gb + b * kWaves) * PPI + sub;
      const bool valid = t < t1;
      if (__ballot(valid) == 0) break;
      float kf[8], vf[8];
      const h8 kh = __builtin_bit_cast(h8, kb[b]), vh = __builtin_bit_cast(h8, vb[b]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[e] = t == c.pos ? kcur[dl * 8 + e] : (float)kh[e];
        vf[e] = t == c.pos ? vcur[dl * 8 + e] : (float)vh[e];
      }
#pragma unroll
      for (int j = 0; j < GP; ++j) {
        if (GP != kSpecGroup && j >= ng) break;
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc = fmaf(q[j][e], kf[e], sc);
        sc = slot_sum<LPP>(sc);
        const float mn = valid ? fmaxf(m[j], sc) : m[j];
        const float al = mn == -INFINITY ? 0.f : exp2f(m[j] - mn);
        const float pv = valid ? exp2f(sc - mn) : 0.f;
        lsum[j] = lsum[j] * al + pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * al + pv * vf[e];
        m[j] = mn;
      }
    }
  }
#endif
  ts_mark(c, 7);  // this wavefront's positions done
  // merge the PPI position slots of the wavefront (lanes dl, dl + LPP, ...)
#pragma unroll
  for (int x = LPP; x < 64; x <<= 1) {
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      const float m2 = __shfl_xor(m[j], x), l2 = __shfl_xor(lsum[j], x);
      const float mn = fmaxf(m[j], m2);
      const float a1 = m[j] == -INFINITY ? 0.f : exp2f(m[j] - mn);
      const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
      lsum[j] = lsum[j] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * a1 + __shfl_xor(o[j][e], x) * a2;
      m[j] = mn;
    }
  }
  // combine the wavefronts: scratch [wave][ng][HD + 2]
  float* scr = c.sm.scratch;
  const int rec = HD + 2;
  if (sub == 0) {
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      if (GP != kSpecGroup && j >= ng) break;
      float* r = scr + (c.wave * ng + j) * rec;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[2 + dl * 8 + e] = o[j][e];
      if (dl == 0) {
        r[0] = m[j];
        r[1] = lsum[j];
      }
    }
  }
  cta_sync(c);
  for (int i = c.tid; i < ng * HD; i += kThreads) {
    const int j = i / HD, dd = i % HD;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, scr[(w * ng + j) * rec]);
    float Lt = 0.f, Ot = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float* r = scr + (w * ng + j) * rec;
        const float al = exp2f(r[0] - M);
        Lt += al * r[1];
        Ot += al * r[2 + dd];
      }
    }
    const int qh = g * G + j0 + j;
    const int64_t po = ((((int64_t)c.e * kp.L + l) * kp.nq + qh) * S + sp);
    const int64_t po1 = ((((int64_t)c.e1 * kp.L + l) * kp.nq + qh) * S + sp);
    stcf(kp.att_o + po * HD + dd, Ot);
    if (sentinel_mode(c)) stc32(kp.att_o + po1 * HD + dd, kSent32);
    if (dd == 0) {
      stcf(kp.att_ml + po * 2, M);
      stcf(kp.att_ml + po * 2 + 1, Lt);
      if (sentinel_mode(c)) {
        stc32(kp.att_ml + po1 * 2, kSent32);
        stc32(kp.att_ml + po1 * 2 + 1, kSent32);
      }
    }
  }
  cta_sync(c);  // scratch reused by the next pass
}

// Query heads per pass: at most 4 (2 for head_dim 256), so the combine fits
// the scratch: kWaves * heads * (HD + 2) floats.
// (pre: K/V groups of the first pass already issued; the DMA-fed pass only)
template <int HD>
__device__ __forceinline__ void att_heads(Cx& c, int l, int g, int sp, int t0, int t1, int G, int pre = 0) {
  constexpr int kMaxPass = HD == 256 ? 2 : 4;
  if (G == 1) {
    att_pass<HD, 1>(c, l, g, sp, 0, 1, t0, t1, G, pre);
  } else if (G == 2 || kMaxPass == 2) {
    for (int j0 = 0; j0 < G; j0 += 2) att_pass<HD, 2>(c, l, g, sp, j0, min(2, G - j0), t0, t1, G, j0 == 0 ? pre : 0);
  } else {
    for (int j0 = 0; j0 < G; j0 += 4) att_pass<HD, 4>(c, l, g, sp, j0, min(4, G - j0), t0, t1, G, j0 == 0 ? pre : 0);
  }
}

// Stage q of kv head g's query group (times log2(e)/sqrt(hd)) and, for the
// split holding the current position, that position's K/V rows (polled: the
// QKV stage writes them) into LDS; ends with a workgroup barrier.
__device__ __forceinline__ void att_stage(Cx& c, int l, int g, bool has_cur, bool first) {
  const KParams& kp = *c.kp;
  const int G = q_group(kp), hd = head_dim(kp);
  const float qscale = kLog2e / __builtin_sqrtf((float)hd);
  float* qs = c.sm.vec;              // [G][hd]
  float* kcur = c.sm.vec + G * hd;   // [hd]
  float* vcur = kcur + hd;           // [hd]
  const float* qsrc = buf_at(kp.q, c.e, l, 0) + g * G * hd;
  {
    // 16-byte polls: G * hd is a multiple of 64 and the group's q 16-byte aligned
    const Rsrc rs = sync_rsrc(qsrc, (uint32_t)(G * hd) * 4u);
    for (int i = c.tid * 4; i < G * hd; i += kThreads * 4) {
      const u4 v = poll_f32x4(c, rs, (uint32_t)i * 4u, OP_ATT, l);
      *(f4*)(qs + i) = f4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])} * qscale;
    }
  }
  if (has_cur && c.tid < hd / 4) {
    // 16-byte polls (8 fp16 values, each checked for the fp16 sentinel): lanes
    // [0, hd/8) read the K row, [hd/8, hd/4) the V row
    const bool isk = c.tid < hd / 8;
    const int i8 = (isk ? c.tid : c.tid - hd / 8) * 8;
    const int64_t row = (((int64_t)l * kp.nkv + g) * kp.max_seq + c.pos) * hd;
    const Rsrc rk = sync_rsrc(kp.kc + row, (uint32_t)hd * 2u), rv = sync_rsrc(kp.vc + row, (uint32_t)hd * 2u);
    u4 v = isk ? ldc128(rk, (uint32_t)i8 * 2u) : ldc128(rv, (uint32_t)i8 * 2u);
    if (sentinel_mode(c)) {
      while (any_sent16(v) && !c.fail) {
        if (expired(c, OP_ATT, l, i8)) {
          c.fail = true;
          break;
        }
        v = isk ? ldc128(rk, (uint32_t)i8 * 2u) : ldc128(rv, (uint32_t)i8 * 2u);
      }
    }
    float* dst = (isk ? kcur : vcur) + i8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[j] & 0xFFFFu));
      dst[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[j] >> 16));
    }
  }
  ts_mark(c, 1);
  cta_sync(c);
  ts_mark(c, 2);
  if (first) mark_ready(c);
}

// DPL fp16 values of one cached K or V row slice, kept as loaded (the
// conversion waits for the load, so it happens after q has been staged).
template <int DPL> struct RawHalves { typedef uint32_t T; };
template <> struct RawHalves<4> { typedef u2 T; };

template <int DPL>
__device__ __forceinline__ typename RawHalves<DPL>::T load_halves(const uint16_t* p) {
  if constexpr (DPL == 1) return (uint32_t)*gp(p);
  else if constexpr (DPL == 2) return *gp((const uint32_t*)p);
  else return *gp((const u2*)p);
}

template <int DPL>
__device__ __forceinline__ float half_at(const typename RawHalves<DPL>::T& r, int k) {
  uint32_t w;
  if constexpr (DPL == 4) w = r[k >> 1];
  else w = r;
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * (k & 1))));
}

// Short split: this wavefront's cached K/V rows are loaded before q is
// polled, so their latency hides behind the wait for the QKV stage.  Loads
// with the default cache policy: a short context's K/V (96 MB for 24 layers
// at 1024 positions) stays in the memory-side cache from token to token
// (nontemporal loads: 458.6 vs 452.6 ms per 512 tokens).
template <int GP, int DPL>
__device__ __forceinline__ void att_short(Cx& c, Ring& ring, int l, int g, int sp, int t0, int t1, int G, bool has_cur, bool first) {
  const KParams& kp = *c.kp;
  const int hd = head_dim(kp);
  typedef typename RawHalves<DPL>::T Raw;
  Raw kr[kPosBatch], vr[kPosBatch];
  const int64_t head_off = ((int64_t)l * kp.nkv + g) * kp.max_seq * hd + c.lane * DPL;
#pragma unroll
  for (int b = 0; b < kPosBatch; ++b) {
    const int t = t0 + c.wave + b * kWaves;
    kr[b] = Raw{};
    vr[b] = Raw{};
    if (t < t1 && t != c.pos) {
      kr[b] = load_halves<DPL>(kp.kc + head_off + (int64_t)t * hd);
      vr[b] = load_halves<DPL>(kp.vc + head_off + (int64_t)t * hd);
    }
  }
  att_stage(c, l, g, has_cur, first);
  const float* kcur = c.sm.vec + G * hd;
  const float* vcur = kcur + hd;
  float kv[kPosBatch][DPL], vv[kPosBatch][DPL];
#pragma unroll
  for (int b = 0; b < kPosBatch; ++b) {
    const bool cur = t0 + c.wave + b * kWaves == c.pos;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      kv[b][k] = cur ? kcur[c.lane * DPL + k] : half_at<DPL>(kr[b], k);
      vv[b][k] = cur ? vcur[c.lane * DPL + k] : half_at<DPL>(vr[b], k);
    }
  }
  for (int j0 = 0; j0 < G; j0 += GP) att_pos_core<GP, DPL>(c, ring, l, g, sp, j0, min(GP, G - j0), t0, t1, G, kv, vv);
}

__device__ __forceinline__ void op_att(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int l = in.layer;
  const int G = q_group(kp), hd = head_dim(kp), S = kp.S;
  const int T = c.pos + 1;
  const int chunk = (T + S - 1) / S;
  counter_wait(c, in.sync_in, in.n_in, OP_ATT, l);
  if (!sentinel_mode(c)) cta_sync(c);
  for (int ui = 0; ui < in.nu; ++ui) {
    const int U = in.u0 + ui, g = U / S, sp = U % S;
    const int t0 = sp * chunk, t1 = min(T, t0 + chunk);
    const bool has_cur = t0 <= c.pos && c.pos < t1;
    if (t1 - t0 <= kShortSplitMax) {
      // short split (at most kPosBatch positions per wavefront): scores of the batch first, then one softmax per head
      const int dpl = hd / 64;
#ifdef MK_SPECIALIZED
      (void)dpl;
      att_short<kSpecGroup, 2>(c, ring, l, g, sp, t0, t1, G, has_cur, ui == 0);
#else
      if (dpl == 1) att_short<8, 1>(c, ring, l, g, sp, t0, t1, G, has_cur, ui == 0);
      else if (dpl == 2) att_short<4, 2>(c, ring, l, g, sp, t0, t1, G, has_cur, ui == 0);
      else att_short<2, 4>(c, ring, l, g, sp, t0, t1, G, has_cur, ui == 0);
#endif
    } else {
#ifdef MK_LONG_DMA
      // the wavefront's first two K/V groups go out before q is polled (their rows are in the
      // cache already) and land while it waits; pulling the split's whole K/V towards L2 there
      // instead was measured slower (it delayed the q polls)
      int pre = 0;
      {
        const KvRing r = kv_ring<128>(c, l, g, t0, t1, G);
        for (; pre < 2 && pre < r.mine; ++pre) kv_issue<128>(c, r, t0, t1, pre);
      }
#else
      // (no prefetch of the split's K/V rows before the wait: pulling them
      // towards L2 first was measured slower at 2048 and 8192 positions)
      const int pre = 0;
#endif
      att_stage(c, l, g, has_cur, ui == 0);
#ifdef MK_SPECIALIZED
      att_heads<128>(c, l, g, sp, t0, t1, G, pre);
#else
      if (hd == 64) att_heads<64>(c, l, g, sp, t0, t1, G);
      else if (hd == 128) att_heads<128>(c, l, g, sp, t0, t1, G);
      else att_heads<256>(c, l, g, sp, t0, t1, G);
#endif
      // the refills QKV left owed go out behind the split's K/V loads (issued after q is staged): 296.4 -> 292.5
      // ms per 256 tokens at an 8192-token context against issuing them right after the q polls
      ring_settle(ring);
    }
    ts_mark(c, 6);
    if (!sentinel_mode(c)) {
      // counter mode: count this finished split of kv head g (release before the count)
      stores_acked();
      cta_sync(c);
      if (c.tid == 0) {
        release_stores();
        __hip_atomic_fetch_add(gp(kp.att_cnt + l * kp.nkv + g), 1u, __ATOMIC_RELAXED, MK_SCOPE);
      }
    }
    if (ui + 1 < in.nu) cta_sync(c);  // the staging and the scratch are reused by the next unit
  }
  // Merge right here, without a reduction stage: the splits of a kv head
  // share its reduce units (query head, kRedDims dims) -- split sp takes
  // units sp, sp + S, ... -- and each waits for the S partials it needs.
  // Every partial of this workgroup is published before it waits for any
  // other, so a workgroup holding several splits of one head cannot wait on
  // itself.  Sentinel mode polls the partials themselves; counter mode waits
  // until all S splits of the head are counted.
  for (int ui = 0; ui < in.nu; ++ui) {
    const int U = in.u0 + ui, g = U / S, sp = U % S;
    if (!sentinel_mode(c) && (ui == 0 || sp == 0)) {
      if (c.tid == 0) {
        const uint32_t* cnt = kp.att_cnt + l * kp.nkv + g;
        const uint32_t target = (uint32_t)S * (uint32_t)(c.step + 1);
        while (!c.fail && __hip_atomic_load(gp(cnt), __ATOMIC_RELAXED, MK_SCOPE) < target) {
          if (expired(c, OP_ATT, l, g)) {
            c.fail = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        acquire_polled();
      }
      cta_sync(c);
    }
    const int nb = hd / kRedDims, units = G * nb;
    for (int v = sp + c.wave * S; v < units; v += S * kWaves) red_unit(c, l, g * G + v / nb, v % nb);
  }
  cta_sync(c);  // the next instruction restages the vector the partials read
  counter_signal(c, in.sync_out);
}

__device__ __forceinline__ void op_oproj(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int l = in.layer;
  counter_wait(c, in.sync_in, in.n_in, OP_OPROJ, l);
  if (!sentinel_mode(c)) cta_sync(c);
  const float* rsrc = l == 0 ? nullptr : buf_at(kp.xm, c.e, l - 1, c.rep);
  const uint16_t* remb = l == 0 ? kp.embed + (int64_t)c.tok * kp.d : nullptr;
  const uint32_t r0 = resid_issue(c, rsrc, remb, in.u0, in.nu);
  stage_vec(c, buf_at(kp.o, c.e, l, c.rep), c.sm.vec, kp.nq * kp.hd, in.kpad, nullptr, OP_OPROJ, l);
  resid_finish(c, r0, rsrc, remb, in.u0, in.nu, OP_OPROJ, l);
  finish_staging(c, 0, false, 0.f);
  const bool staged = staged_rows(in);
  gemv_dispatch(c, ring, in, c.sm.vec, 1.f, [&](int u, float y, float) {
    const float v = c.sm.resid[u] + y;
    if (!staged) publish(c, kp.xa, l, in.u0 + u, v);
    else if (c.lane == 0) c.sm.resid[u] = v;
  });
  if (staged) {
    cta_sync(c);
    publish_rows(c, kp.xa, c.e, l, in.u0, in.nu, c.sm.resid, true);
  }
  ring_settle(ring);
  counter_signal(c, in.sync_out);
}

__device__ __forceinline__ void op_upgate(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int l = in.layer;
  counter_wait(c, in.sync_in, in.n_in, OP_UPGATE, l);
  if (!sentinel_mode(c)) cta_sync(c);
  const uint16_t* g2 = kp.norms + ((int64_t)l * 2 + 1) * kp.d;
  const float ss = stage_vec(c, buf_at(kp.xa, c.e, l, c.rep), c.sm.vec, kp.d, in.kpad, g2, OP_UPGATE, l);
  const float scale = finish_staging(c, kp.d, true, ss);
  const bool staged = staged_rows(in);
  gemv_dispatch(c, ring, in, c.sm.vec, scale, [&](int u, float gt, float up) {
    const float silu = gt / (1.0f + __expf(-gt));
    if (!staged) publish(c, kp.m, l, in.u0 + u, silu * up);
    else if (c.lane == 0) c.sm.resid[u] = silu * up;
  });
  if (staged) {
    cta_sync(c);
    publish_rows(c, kp.m, c.e, l, in.u0, in.nu, c.sm.resid, true);
  }
  ring_settle(ring);
  counter_signal(c, in.sync_out);
}

__device__ __forceinline__ void op_down(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int l = in.layer;
  counter_wait(c, in.sync_in, in.n_in, OP_DOWN, l);
  if (!sentinel_mode(c)) cta_sync(c);
  const float* rsrc = buf_at(kp.xa, c.e, l, c.rep);
  const uint32_t r0 = resid_issue(c, rsrc, nullptr, in.u0, in.nu);
  stage_vec(c, buf_at(kp.m, c.e, l, c.rep), c.sm.vec, kp.f, in.kpad, nullptr, OP_DOWN, l);
  resid_finish(c, r0, rsrc, nullptr, in.u0, in.nu, OP_DOWN, l);
  finish_staging(c, 0, false, 0.f);
  const bool staged = staged_rows(in);
  gemv_dispatch(c, ring, in, c.sm.vec, 1.f, [&](int u, float y, float) {
    const float v = c.sm.resid[u] + y;
    if (!staged) publish(c, kp.xm, l, in.u0 + u, v);
    else if (c.lane == 0) c.sm.resid[u] = v;
  });
  if (staged) {
    cta_sync(c);
    publish_rows(c, kp.xm, c.e, l, in.u0, in.nu, c.sm.resid, true);
  }
  ring_settle(ring);
  counter_signal(c, in.sync_out);
}

// Argmax key: order-preserving map of the logit in the high word, the
// complemented row index in the low word (max key = max logit, lowest index).
__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
  uint32_t b = __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t b = (uint32_t)(key >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// ---------------------------------------------------------------- top-k sampling
// Keys order logits like the greedy argmax (larger logit first, equal logits
// by smaller id); every real key is > 1, and 1 marks an empty entry.
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src_lane) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src_lane), hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src_lane);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = shfl_u64(v, lane_id() ^ off);
    v = v > o ? v : o;
  }
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Insert a key (the same value in every lane) into a wavefront's list of its
// K largest keys, held in descending order by lanes 0..K-1.
__device__ __forceinline__ void topk_insert(uint64_t& mine, uint64_t key, int K) {
  const int lane = lane_id();
  const uint64_t gt = __ballot(lane < K && key > mine);  // a suffix of lanes [p, K)
  if (gt == 0) return;
  const int p = __builtin_ctzll(gt);
  const uint64_t prev = shfl_u64(mine, lane > 0 ? lane - 1 : 0);
  if (lane == p) mine = key;
  else if (lane > p && lane < K) mine = prev;
}

// The K largest of the keys every lane holds in v[0..M) (consumed), in
// descending order in lanes 0..K-1 (1 where fewer than K real keys exist).
template <int M>
__device__ __forceinline__ uint64_t wave_topk(uint64_t (&v)[M], int K) {
  uint64_t out = 1;
  for (int j = 0; j < K; ++j) {
    uint64_t m = 1;
#pragma unroll
    for (int i = 0; i < M; ++i) m = v[i] > m ? v[i] : m;
    const uint64_t w = wave_max_u64(m);
    if (w <= 1) break;
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (v[i] == w) v[i] = 1;  // keys are distinct (each carries its row)
    if (lane_id() == j) out = w;
  }
  return out;
}

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC11): first output word for the counter
// (ctr, 0, 0, 0) and the key (k0, k1).  A round multiplies words 0 and 2 by
// the two round constants and recombines the 64-bit products with words 1, 3
// and the key; the key is advanced by the two Weyl increments between rounds.
__device__ __forceinline__ uint32_t philox_word0(uint32_t ctr, uint32_t k0, uint32_t k1) {
  uint32_t x0 = ctr, x1 = 0u, x2 = 0u, x3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * x0, hi0 = __umulhi(0xD2511F53u, x0);
    const uint32_t lo1 = 0xCD9E8D57u * x2, hi1 = __umulhi(0xCD9E8D57u, x2);
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  return x0;
}

__device__ __forceinline__ void op_lmhead(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int L = kp.L;
  counter_wait(c, in.sync_in, in.n_in, OP_LMHEAD, L);
  if (!sentinel_mode(c)) cta_sync(c);
  uint64_t best = 1;  // below every real key
  const int K = kp.top_k > 1 ? kp.top_k : 1;
  uint64_t wl = 1;    // sampling: the workgroup's K largest keys in lanes 0..K-1 of wavefront 0
  if (in.nu > 0) {
    const uint16_t* gf = kp.norms + (int64_t)L * 2 * kp.d;
    const float ss = stage_vec(c, buf_at(kp.xm, c.e, L - 1, c.rep), c.sm.vec, kp.d, in.kpad, gf, OP_LMHEAD, L);
    const float scale = finish_staging(c, kp.d, true, ss);
    float* lo = kp.logits ? kp.logits + (int64_t)c.step * kp.V : nullptr;
    float bv = -INFINITY;
    int bi = -1;
    bool nan = false;
    uint64_t mine = 1;  // sampling: this wavefront's K largest keys, lane j the j-th
    gemv_dispatch(c, ring, in, c.sm.vec, scale, [&](int u, float y, float) {
      const int row = in.u0 + u;
      if (lo && c.lane == 0) *gp(lo + row) = y;
      if (y != y) {
        nan = true;
      } else {
        if (bi < 0 || y > bv || (y == bv && row < bi)) {
          bv = y;
          bi = row;
        }
        if (K > 1) topk_insert(mine, argmax_key(y, row), K);
      }
    });
    if (nan && c.lane == 0) raise_fault(c, -8, OP_LMHEAD, L, c.step);
    if (c.lane == 0) c.sm.keys[c.wave] = bi >= 0 ? argmax_key(bv, bi) : 1;
    cta_sync(c);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) best = max(best, c.sm.keys[w]);
    if (K > 1) {
      // the workgroup's K largest: wavefront lists through the scratch, merged by wavefront 0
      uint64_t* lists = (uint64_t*)c.sm.scratch;  // [kWaves][K]
      if (c.lane < K) lists[c.wave * K + c.lane] = mine;
      cta_sync(c);
      if (c.wave == 0) {
        static_assert(kWaves * kMaxTopK <= 128, "two list entries per lane");
        uint64_t v[2] = {c.lane < kWaves * K ? lists[c.lane] : 1, c.lane + 64 < kWaves * K ? lists[c.lane + 64] : 1};
        wl = wave_topk<2>(v, K);
      }
    }
  }
  // re-arm the slot for the step after next, then one release fence per step
  // orders this step's stores (KV cache, re-arms) before the key.
  uint64_t* slot = kp.lmp + c.e * kp.lmp_es + in.slot;
  uint64_t* slot1 = kp.lmp + c.e1 * kp.lmp_es + in.slot;
  if (sentinel_mode(c) && c.wave == 0 && c.lane < kp.R) stc64(slot1 + c.lane * kp.lmp_rs, kSent64);
  uint64_t* list = kp.lmk + c.e * kp.lmk_es + (int64_t)in.slot * kMaxTopK;
  uint64_t* list1 = kp.lmk + c.e1 * kp.lmk_es + (int64_t)in.slot * kMaxTopK;
  if (K > 1 && sentinel_mode(c) && c.wave == 0 && c.lane < K)
    for (int r = 0; r < kp.R; ++r) stc64(list1 + r * kp.lmk_rs + c.lane, kSent64);
  stores_acked();
  cta_sync(c);
  if (c.wave == 0) {
    release_stores();
    if (c.lane < kp.R) stc64(slot + c.lane * kp.lmp_rs, best);
    if (K > 1 && c.lane < K)
      for (int r = 0; r < kp.R; ++r) stc64(list + r * kp.lmk_rs + c.lane, wl);
    if (!sentinel_mode(c)) {
      // counter mode: the keys themselves must be out before the count says so
      release_stores();
      if (c.lane == 0) __hip_atomic_fetch_add(gp(kp.counters + in.sync_out), 1u, __ATOMIC_RELAXED, MK_SCOPE);
    }
  }
  ring_settle(ring);
}

// Sampling instead of the argmax: every workgroup merges the per-workgroup
// top-K lists (polled like the argmax keys) into the global K largest keys,
// then draws the token by the inverse-CDF rule with a Philox uniform.  The
// arithmetic is the same in every workgroup, so all draw the same token.
__device__ __forceinline__ void op_sample_all(Cx& c, const Ins& in) {
  const KParams& kp = *c.kp;
  const int K = kp.top_k, n = in.nu * K;
  const uint64_t* src = kp.lmk + c.e * kp.lmk_es + c.rep * kp.lmk_rs;  // [slot][kMaxTopK]
  constexpr int kPer = 8;
  uint64_t wl = 1;  // this wavefront's running K largest
  for (int base = 0; base < n; base += kThreads * kPer) {
    uint64_t v[kPer + 1];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = base + c.tid + j * kThreads;
      v[j] = i < n ? ldc64(src + (i / K) * kMaxTopK + i % K) : 1;
    }
    if (sentinel_mode(c)) {
      for (;;) {
        bool pending = false;
#pragma unroll
        for (int j = 0; j < kPer; ++j) pending |= v[j] == kSent64;
        if (!pending || c.fail) break;
        if (expired(c, OP_ARGMAX, kp.L, base)) {
          c.fail = true;
          break;
        }
        poll_pause(c);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int i = base + c.tid + j * kThreads;
          if (v[j] == kSent64) v[j] = ldc64(src + (i / K) * kMaxTopK + i % K);
        }
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (v[j] == kSent64) v[j] = 1;  // only on an aborted run
    }
    v[kPer] = wl;
    wl = wave_topk<kPer + 1>(v, K);
  }
  uint64_t* lists = (uint64_t*)c.sm.scratch;  // [kWaves][K]
  if (c.lane < K) lists[c.wave * K + c.lane] = wl;
  cta_sync(c);
  mark_ready(c);
  if (c.wave == 0) {
    acquire_polled();
    uint64_t v[2] = {c.lane < kWaves * K ? lists[c.lane] : 1, c.lane + 64 < kWaves * K ? lists[c.lane + 64] : 1};
    const uint64_t key = wave_topk<2>(v, K);
    // weights exp((z_j - z_0) / T) of the candidates in order; running sums in that order
    const uint32_t top_hi = __builtin_amdgcn_readfirstlane((uint32_t)(key >> 32));
    const uint32_t top_lo = __builtin_amdgcn_readfirstlane((uint32_t)key);
    const uint64_t top = ((uint64_t)top_hi << 32) | top_lo;  // lane 0: the largest logit
    const float z0 = key_value(top);
    const float w = c.lane < K && key > 1 ? exp2f((key_value(key) - z0) * kp.inv_temp * kLog2e) : 0.f;
    const uint32_t word = philox_word0((uint32_t)c.pos, kp.seed_lo, kp.seed_hi);
    const float u = (float)(word >> 8) * 0x1p-24f;
    float total = 0.f;
    for (int j = 0; j < K; ++j) total += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
    const float target = u * total;
    float cum = 0.f;
    int pick = K - 1;
    for (int j = 0; j < K; ++j) {
      cum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
      if (cum > target) {
        pick = j;
        break;
      }
    }
    const int id = key_index(key);
    const int tok = __builtin_amdgcn_readlane(id, pick);
    if (c.lane == 0) c.sm.misc[1] = (uint32_t)tok;
  }
  cta_sync(c);
  int tok = __builtin_amdgcn_readfirstlane((int)c.sm.misc[1]);
  if (tok < 0 || tok >= kp.V) tok = 0;  // only on an aborted run
  if (c.cta == 0 && c.tid == 0) *gp(kp.tokens + c.step) = tok;
  c.tok = tok;
}

// Poll M 8-byte keys per lane (null address: no key, reads as 1) until none is
// the sentinel; every pending key is re-polled in one batch.
template <int M>
__device__ __forceinline__ void poll_keys(Cx& c, uint64_t (&v)[M], const uint64_t* const (&a)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) v[i] = a[i] ? ldc64(a[i]) : 1;
  if (!sentinel_mode(c)) return;
  for (;;) {
    bool pending = false;
#pragma unroll
    for (int i = 0; i < M; ++i) pending |= v[i] == kSent64;
    if (!pending || c.fail) break;
    if (expired(c, OP_ARGMAX, c.kp->L, -1)) {
      c.fail = true;
      break;
    }
    poll_pause(c);
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (v[i] == kSent64) v[i] = ldc64(a[i]);
  }
#pragma unroll
  for (int i = 0; i < M; ++i)
    if (v[i] == kSent64) v[i] = 1;  // only on an aborted run
}

// Sampling with at most 256 workgroup lists: the global K largest keys all come
// from the workgroups whose own maximum is among the K largest maxima (any other
// workgroup has K larger keys elsewhere), so wavefront 0 first polls the
// per-workgroup maxima (the argmax keys), picks the K workgroups with the
// largest ones, then polls only their K lists (K*K <= 256 keys) and merges them.
__device__ __forceinline__ void op_sample(Cx& c, const Ins& in) {
  const KParams& kp = *c.kp;
  const int K = kp.top_k, nslot = in.nu;
  if (nslot > 256) {
    op_sample_all(c, in);
    return;
  }
  if (c.wave == 0) {
    const uint64_t* maxk = kp.lmp + c.e * kp.lmp_es + c.rep * kp.lmp_rs;  // [slot]
    const uint64_t* lists = kp.lmk + c.e * kp.lmk_es + c.rep * kp.lmk_rs;  // [slot][kMaxTopK]
    uint64_t v[4];
    const uint64_t* a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = c.lane + 64 * i;
      a[i] = sl < nslot ? maxk + sl : nullptr;
    }
    poll_keys<4>(c, v, a);
    // lane j: slot of the j-th largest maximum (slot 0 where fewer than K exist)
    int sel = 0;
    for (int j = 0; j < K; ++j) {
      uint64_t m = 1;
      int mi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (v[i] > m) {
          m = v[i];
          mi = i;
        }
      const uint64_t w = wave_max_u64(m);
      if (w <= 1) break;
      const int owner = (int)__builtin_ctzll(__ballot(m == w));
      const int slot = __builtin_amdgcn_readlane(c.lane + 64 * mi, owner);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c.lane == owner && i == mi) v[i] = 1;
      if (c.lane == j) sel = slot;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = c.lane + 64 * i;  // key q: element q % K of the (q / K)-th selected list
      const int sl = __shfl(sel, q < K * K ? q / K : 0);
      a[i] = q < K * K ? lists + (int64_t)sl * kMaxTopK + q % K : nullptr;
    }
    poll_keys<4>(c, v, a);
    mark_ready(c);
    acquire_polled();
    const uint64_t key = wave_topk<4>(v, K);  // lane j: the j-th largest key
    // weights exp((z_j - z_0) / T) of the candidates in order; running sums in that order
    const uint32_t top_hi = __builtin_amdgcn_readfirstlane((uint32_t)(key >> 32));
    const uint32_t top_lo = __builtin_amdgcn_readfirstlane((uint32_t)key);
    const uint64_t top = ((uint64_t)top_hi << 32) | top_lo;  // lane 0: the largest logit
    const float z0 = key_value(top);
    const float w = c.lane < K && key > 1 ? exp2f((key_value(key) - z0) * kp.inv_temp * kLog2e) : 0.f;
    const uint32_t word = philox_word0((uint32_t)c.pos, kp.seed_lo, kp.seed_hi);
    const float u = (float)(word >> 8) * 0x1p-24f;
    float total = 0.f;
    for (int j = 0; j < K; ++j) total += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
    const float target = u * total;
    float cum = 0.f;
    int pick = K - 1;
    for (int j = 0; j < K; ++j) {
      cum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
      if (cum > target) {
        pick = j;
        break;
      }
    }
    const int id = key_index(key);
    const int tok = __builtin_amdgcn_readlane(id, pick);
    if (c.lane == 0) c.sm.misc[1] = (uint32_t)tok;
  }
  cta_sync(c);
  int tok = __builtin_amdgcn_readfirstlane((int)c.sm.misc[1]);
  if (tok < 0 || tok >= kp.V) tok = 0;  // only on an aborted run
  if (c.cta == 0 && c.tid == 0) *gp(kp.tokens + c.step) = tok;
  c.tok = tok;
}

__device__ __forceinline__ void op_argmax(Cx& c, const Ins& in) {
  const KParams& kp = *c.kp;
  counter_wait(c, in.sync_in, in.n_in, OP_ARGMAX, kp.L);
  if (!sentinel_mode(c)) cta_sync(c);
  // Failure-path test (armed by the host for one launch): wait for a word that
  // is never written, so this wait's watchdog fires and every other workgroup
  // leaves its own waits through the abort flag.
  if (c.step == 0 && c.cta == kp.stall_cta && c.tid == 0) (void)poll_f32(c, (const float*)kp.stall_word, OP_ARGMAX, kp.L);
  if (kp.top_k > 1) {
    op_sample(c, in);
    return;
  }
  const uint64_t* src = kp.lmp + c.e * kp.lmp_es + c.rep * kp.lmp_rs;
  uint64_t k = 0;
  for (int i = c.tid; i < in.nu; i += kThreads) {
    uint64_t v = ldc64(src + i);
    if (sentinel_mode(c)) {
      while (v == kSent64 && !c.fail) {
        if (expired(c, OP_ARGMAX, kp.L, i)) {
          c.fail = true;
          break;
        }
        poll_pause(c);
        v = ldc64(src + i);
      }
    }
    k = max(k, v);
  }
  // workgroup max
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off);
    k = max(k, o);
  }
  if (c.lane == 0) c.sm.keys[c.wave] = k;
  cta_sync(c);
  mark_ready(c);
  // one acquire (cache invalidation) for the workgroup, after every wavefront's polls
  if (c.wave == 0) acquire_polled();
  cta_sync(c);
  uint64_t best = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) best = max(best, c.sm.keys[w]);
  int tok = __builtin_amdgcn_readfirstlane((int)(0xFFFFFFFFu - (uint32_t)best));
  if (tok < 0 || tok >= kp.V) tok = 0;  // only on an aborted run
  if (c.cta == 0 && c.tid == 0) *gp(kp.tokens + c.step) = tok;
  c.tok = tok;
}

__device__ __forceinline__ void op_chain(Cx& c, Ring& ring, const Ins& in) {
  const KParams& kp = *c.kp;
  const int i = in.layer, n = kp.chain_n;
  counter_wait(c, in.sync_in, in.n_in, OP_CHAIN, i);
  if (!sentinel_mode(c)) cta_sync(c);
  if (i == 0) {
    for (int k = c.tid * 4; k < in.kpad; k += kThreads * 4)
      *(f4*)(c.sm.vec + k) = k < n ? *gp((const f4*)(kp.x0 + k)) : f4{0.f, 0.f, 0.f, 0.f};
  } else {
    stage_vec(c, buf_at(kp.y, 0, i - 1, c.rep), c.sm.vec, n, in.kpad, nullptr, OP_CHAIN, i);
  }
  finish_staging(c, 0, false, 0.f);
  const bool staged = staged_rows(in);
  gemv_dispatch(c, ring, in, c.sm.vec, 1.f, [&](int u, float y, float) {
    const float t = tanhf(y);
    if (!staged) {
      if (c.lane < kp.R) stcf(buf_at(kp.y, 0, i, c.lane) + in.u0 + u, t);
    } else if (c.lane == 0) {
      c.sm.resid[u] = t;
    }
  });
  if (staged) {
    cta_sync(c);
    publish_rows(c, kp.y, 0, i, in.u0, in.nu, c.sm.resid, false);
  }
  ring_settle(ring);
  counter_signal(c, in.sync_out);
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void MK_MONOKERNEL(const KParams* __restrict__ kpp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const KParams& kp = *kpp;
  Cx c;
  c.kp = kpp;
  c.cta = blockIdx.x;
  c.tid = threadIdx.x;
  c.lane = lane_id();
  c.wave = wave_id();
  c.xcc = xcc_id();
  c.rep = c.xcc % kp.R;
  c.fail = false;
  c.deadline = 0;
  c.poll_iters = 0;
  c.flag_parity = 0;
  c.pc = 0;
  // LDS carve-up (must match lds_bytes_for on the host)
  c.sm.base = smem;
  const uint32_t ring_base = (uint32_t)(uintptr_t)smem;
  c.sm.vec = (float*)(smem + kWaves * kRing * 1024);
  c.sm.scratch = c.sm.vec + kp.vec_floats;
  c.sm.resid = c.sm.scratch + kScratchFloats;
  uint8_t* small = (uint8_t*)(c.sm.resid + kResidRows);
  c.sm.flags = (uint32_t*)(small + kOffFlags);
  c.sm.wsum = (float*)(small + kOffWsum);
  c.sm.keys = (uint64_t*)(small + kOffKeys);
  c.sm.misc = (uint32_t*)(small + kOffMisc);

  Ring ring;
  {
    const int wi = c.cta * kWaves + c.wave;
    ring.lds = __builtin_amdgcn_readfirstlane(ring_base + c.wave * kRing * 1024);
    ring.n = __builtin_amdgcn_readfirstlane((uint32_t)kp.wave_n[wi]);
    ring.g = (const uint8_t*)uniform_ptr(kp.stream + kp.wave_off[wi] * 1024);
    ring.issue = 0;
    ring.slot = 0;
    ring.owed = 0;
    ring_start(ring);
  }

  // drop any line an earlier kernel (e.g. the sentinel fill) left in this XCD's L2
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // values every lane shares: keep them in scalar registers, or the whole
  // instruction loop (and the switch on the opcode) becomes divergent code
  const int beg = __builtin_amdgcn_readfirstlane(kp.ins_off[c.cta]);
  const int end = __builtin_amdgcn_readfirstlane(kp.ins_off[c.cta + 1]);
  c.tok = __builtin_amdgcn_readfirstlane(kp.forced ? kp.forced[0] : kp.first_token);
  uint32_t* trace = nullptr;
  for (int step = 0; step < kp.n_steps; ++step) {
    c.step = step;
    c.pos = kp.pos0 + step;
    c.e = step % 3;
    c.e1 = (step + 1) % 3;
    const bool tr = kp.trace && step < kp.trace_steps;
    if (tr) trace = kp.trace + (((int64_t)c.cta * kp.trace_steps + step) * kp.max_ins) * 8;
    for (int pc = beg; pc < end; ++pc) {
      c.pc = pc - beg;
      const Ins in = load_ins(kp.ins + pc);
      c.deadline = 0;  // every wait gets its own watchdog budget
      c.poll_iters = 0;
      uint64_t t_wait = 0;
      if (tr) {
        t_wait = __builtin_amdgcn_s_memrealtime();
        if (c.tid == 0) c.sm.misc[0] = 0;
      }
      ts_mark(c, 0);
      switch (in.op) {
        case OP_QKV: op_qkv(c, ring, in); break;
        case OP_ATT: op_att(c, ring, in); break;
        case OP_OPROJ: op_oproj(c, ring, in); break;
        case OP_UPGATE: op_upgate(c, ring, in); break;
        case OP_DOWN: op_down(c, ring, in); break;
        case OP_LMHEAD: op_lmhead(c, ring, in); break;
        case OP_ARGMAX: op_argmax(c, in); break;
        case OP_CHAIN: op_chain(c, ring, in); break;
        default: break;
      }
      // thread 0 is past the op's last output stores (issued, not yet acknowledged): the journal's
      // publish time, before the progress store and the failure vote
      uint64_t t_pub = 0;
      if (tr && c.tid == 0) t_pub = __builtin_amdgcn_s_memrealtime();
      ts_mark(c, 3);
      // written through (not left dirty in L2), so the step's release fence finds nothing to write back
      if (c.tid == 0) stc32(kp.progress + c.cta, ((uint32_t)step << 16) | (uint32_t)(c.pc + 1));
      if (cta_failed(c)) goto done;
      ts_mark(c, 4);
      if (tr && c.tid == 0) {
        const uint64_t t_done = __builtin_amdgcn_s_memrealtime();
        MK_GLOBAL uint32_t* r = gp(trace + (int64_t)c.pc * 8);
        r[0] = (uint32_t)c.cta;
        r[1] = (uint32_t)step;
        r[2] = (uint32_t)c.pc;
        r[3] = (uint32_t)in.op | ((uint32_t)(in.layer & 0xFFFF) << 8) | ((uint32_t)(c.xcc & 0x7F) << 24) | (1u << 31);
        r[4] = (uint32_t)t_wait;
        r[5] = c.sm.misc[0] ? c.sm.misc[0] - (uint32_t)t_wait : 0u;
        r[6] = (uint32_t)(t_done - t_wait);
        r[7] = (uint32_t)(t_pub - t_wait);
      }
    }
    if (kp.forced && step + 1 < kp.n_steps) c.tok = __builtin_amdgcn_readfirstlane(kp.forced[step + 1]);
  }
done:
  asm volatile("s_waitcnt vmcnt(0)");
}

#ifndef MK_SPECIALIZED
// ---------------------------------------------------------------- helper kernels
// Fill n 32-bit words with a value.
__global__ void mk_fill32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// Re-arm the KV-cache positions [p0, p1) of every layer and kv head.
__global__ void mk_fill_kv(uint16_t* kc, uint16_t* vc, int64_t rows, int max_seq, int hd, int p0, int p1) {
  const int64_t per_row = (int64_t)(p1 - p0) * hd;
  const int64_t n = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row, k = i % per_row;
    const int64_t o = r * max_seq * hd + (int64_t)p0 * hd + k;
    kc[o] = kSent16;
    vc[o] = kSent16;
  }
}

// Gather weights into wavefront streams: chunk i copies `valid` fp16 values
// from src[i] and zero-fills the rest of its 512.
struct GatherDesc {
  const uint16_t* src;
  int32_t valid;
  int32_t pad;
};
__global__ void mk_gather(uint16_t* dst, const GatherDesc* desc, int64_t n_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t w = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t i = w; i < n_chunks; i += nw) {
    const GatherDesc d = desc[i];
    uint16_t* o = dst + i * kChunkHalfs + lane * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int col = lane * 8 + k;
      o[k] = col < d.valid ? d.src[col] : (uint16_t)0;
    }
  }
}

// Count words equal to the fp32 sentinel (or the fp16 one, for KV ranges).
__global__ void mk_count32(const uint32_t* p, int64_t n, uint32_t v, unsigned long long* out) {
  unsigned long long cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) cnt += p[i] == v;
  atomicAdd(out, cnt);
}
__global__ void mk_count_kv(const uint16_t* kc, const uint16_t* vc, int64_t rows, int max_seq, int hd, int p0, int p1,
                            unsigned long long* out) {
  const int64_t per_row = (int64_t)(p1 - p0) * hd;
  const int64_t n = rows * per_row;
  unsigned long long cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row, k = i % per_row;
    const int64_t o = r * max_seq * hd + (int64_t)p0 * hd + k;
    cnt += (kc[o] == kSent16) + (vc[o] == kSent16);
  }
  atomicAdd(out, cnt);
}

// Count 64-bit words equal to v among the first `width` words of every group
// of `stride` (width == stride: every word).
__global__ void mk_count64(const uint64_t* p, int64_t n, int stride, int width, uint64_t v, unsigned long long* out) {
  unsigned long long cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    cnt += (i % stride) < width && p[i] == v;
  atomicAdd(out, cnt);
}

// ---------------------------------------------------------------- allocation-free scratch
// Device memory of the allocation-free entry point mk_count_sentinels_noalloc:
// its sentinel counter lives here instead of in a per-call allocation.  Each
// GPU holds its own copy until the process ends.  In host code this name is
// not a device address: host code reaches the array only through the address
// hipGetSymbolAddress gives on that device (mk_scratch_address below).
constexpr int kScratchWords = 32;  // 256 bytes; the counter takes the first 8
static __device__ __align__(256) unsigned long long scratch[kScratchWords];

// ---------------------------------------------------------------- calibration probes
// An empty kernel: launch overhead.
__global__ void mk_probe_empty() {}

// `rounds` naive grid barriers: every workgroup's first thread releases, adds 1
// to one counter and polls it (system scope) until it reaches round x grid --
// the pattern the atomic-counter path pays per stage.  Workgroup 0 records the
// elapsed device-clock ticks in out[0]; a deadline ends every wait, and out[1]
// is set when one expired.
__global__ __launch_bounds__(64) void mk_probe_barrier_k(uint32_t* counter, int rounds, uint64_t deadline_ticks,
                                                          uint64_t* out) {
  __shared__ int failed;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) failed = 0;
  __syncthreads();
  for (int r = 0; r < rounds; ++r) {
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(gp(counter), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const uint32_t target = (uint32_t)(r + 1) * gridDim.x;
      while (__hip_atomic_load(gp(counter), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < target) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > deadline_ticks) {
          failed = 1;
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (failed) break;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = __builtin_amdgcn_s_memrealtime() - t0;
    out[1] = (uint64_t)failed;
  }
}

// ---------------------------------------------------------------- host-side launch wrappers
// Internal to the library (not part of the C ABI in include/mk.h).
#endif  // !MK_SPECIALIZED

#define MK_INTERNAL __attribute__((visibility("hidden")))
#ifdef MK_SPECIALIZED
extern "C" {
MK_INTERNAL hipError_t MK_SPEC_LAUNCH(const KParams* kp_dev, int grid, int lds_bytes, hipStream_t s) {
  hipLaunchKernelGGL(MK_MONOKERNEL, dim3(grid), dim3(kThreads), lds_bytes, s, kp_dev);
  return hipGetLastError();
}
MK_INTERNAL hipError_t MK_SPEC_ATTR(int lds_bytes, int* occupancy) {
  hipError_t e = hipFuncSetAttribute((const void*)MK_MONOKERNEL, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, MK_MONOKERNEL, kThreads, lds_bytes);
}
}
#else
extern "C" {
// kp_dev: the parameters, already copied to device memory.
MK_INTERNAL hipError_t mk_launch_monokernel(const KParams* kp_dev, int grid, int lds_bytes, hipStream_t s) {
  hipLaunchKernelGGL(mk_monokernel, dim3(grid), dim3(kThreads), lds_bytes, s, kp_dev);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_kernel_attributes(int lds_bytes, int* occupancy) {
  hipError_t e = hipFuncSetAttribute((const void*)mk_monokernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, mk_monokernel, kThreads, lds_bytes);
}
MK_INTERNAL hipError_t mk_launch_fill32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(mk_fill32, dim3(blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_launch_fill_kv(uint16_t* kc, uint16_t* vc, int64_t rows, int max_seq, int hd, int p0, int p1, hipStream_t s) {
  if (p1 <= p0) return hipSuccess;
  hipLaunchKernelGGL(mk_fill_kv, dim3(2048), dim3(256), 0, s, kc, vc, rows, max_seq, hd, p0, p1);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_launch_gather(uint16_t* dst, const void* desc, int64_t n_chunks, hipStream_t s) {
  if (n_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_gather, dim3(4096), dim3(256), 0, s, dst, (const GatherDesc*)desc, n_chunks);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_launch_probe_empty(hipStream_t s) {
  hipLaunchKernelGGL(mk_probe_empty, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_launch_probe_barrier(uint32_t* counter, int rounds, uint64_t deadline_ticks, uint64_t* out,
                                               int grid, hipStream_t s) {
  hipLaunchKernelGGL(mk_probe_barrier_k, dim3(grid), dim3(64), 0, s, counter, rounds, deadline_ticks, out);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_probe_barrier_occupancy(int* occupancy) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, mk_probe_barrier_k, 64, 0);
}
MK_INTERNAL hipError_t mk_launch_count32(const uint32_t* p, int64_t n, uint32_t v, unsigned long long* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_count32, dim3(1024), dim3(256), 0, s, p, n, v, out);
  return hipGetLastError();
}
MK_INTERNAL hipError_t mk_launch_count64(const uint64_t* p, int64_t n, int stride, int width, uint64_t v,
                                         unsigned long long* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_count64, dim3(256), dim3(256), 0, s, p, n, stride, width, v, out);
  return hipGetLastError();
}
// Device address and size of `scratch` on `device`: looked up once per device
// (with that device current) and kept for later calls.
MK_INTERNAL hipError_t mk_scratch_address(int device, void** out, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) (void)hipSetDevice(cur);  // best effort: the caller's device back
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *out = addr[device];
  *bytes = sizeof(scratch);
  return hipSuccess;
}
MK_INTERNAL hipError_t mk_launch_count_kv(const uint16_t* kc, const uint16_t* vc, int64_t rows, int max_seq, int hd, int p0, int p1,
                              unsigned long long* out, hipStream_t s) {
  if (p1 <= p0) return hipSuccess;
  hipLaunchKernelGGL(mk_count_kv, dim3(1024), dim3(256), 0, s, kc, vc, rows, max_seq, hd, p0, p1, out);
  return hipGetLastError();
}
}
#endif  // MK_SPECIALIZED
