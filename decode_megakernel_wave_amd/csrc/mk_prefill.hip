// mk_prefill.hip -- prompt prefill for gfx950 (MI355X): MFMA GEMM tiles and
// causal attention tiles in one persistent launch.
//
// "7 - AMD et le monokernel" (section 7.1) has one persistent kernel run the
// prompt as well as the decode steps.  A prompt of P tokens is a batch of P
// positions: every projection becomes a [P x K] x [K x N] product, which is
// what the matrix cores are for, while the decode step's batch-1 products
// stay GEMVs on the vector units.  This launch computes, for positions
// 0..P-1 of a prompt, every layer of the decoder and writes each position's
// K and V into the cache; the caller then runs the prompt's last token
// through the decode monokernel, which picks the first generated token.
//
// Stages per layer, separated by grid barriers (counter + release/acquire):
//   QKV   [P x d](RMSNorm) x Wqkv^T -> q (fp32, rotated), K and V (fp16 cache)
//   ATT   causal attention of every query head over positions 0..p
//   OPROJ x += O Wo^T
//   UPGATE m = silu((RMSNorm x) Wg^T) * ((RMSNorm x) Wu^T)
//   DOWN  x += m Wd^T
// Activations keep fp32 semantics on fp16 matrix cores: each fp32 operand a
// is split into hi = fp16(a) and lo = fp16(a - hi), and a.w = hi.w + lo.w is
// two MFMAs with fp32 accumulation (fp16 x fp16 products are exact in fp32).
// The RMSNorm is folded into the GEMM: the tile multiplies x by the gain
// while staging it and scales each output row by 1/rms(x) at the end, the
// sum of squares accumulating from the same loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"
#include "mk_layout.h"

using namespace mk;

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPT = 512;               // threads per workgroup
constexpr int kPW = kPT / 64;          // wavefronts per workgroup
constexpr int kTM = 128;               // GEMM tile: rows (positions)
constexpr int kTNmax = 256;            // GEMM tile: weight rows, 128 or 256 (64 or 128 units of two rows)
constexpr int kTK = 32;                // K per pipeline step (two MFMA steps of 16)
// LDS of a GEMM tile: kNst stages of operands as the DMA leaves them (A hi and
// A lo [128 rows][32 halves], B [TN rows][32 halves], each row's 16-byte
// chunks XOR-swizzled), the row scales, a flag word, then the work-queue slot.
constexpr int kNstMax = 4;                        // stages of the widest tile
constexpr int kOpA = kTM * kTK * 2;               // A hi or A lo of one step: 8 KB
constexpr int stage_bytes(int tn) { return 2 * kOpA + tn * kTK * 2; }
constexpr int kRsOff = kNstMax * stage_bytes(kTNmax);
constexpr int kFlagOff = kRsOff + kTM * 4;
constexpr int kGemmLdsBytes = kFlagOff + 16;
// The work-queue slot a workgroup reads its claimed tile from, past every
// stage's own LDS use.
constexpr int kClaimOff = kGemmLdsBytes;
static_assert(kClaimOff + 16 <= 160 * 1024, "prefill LDS exceeds a CU's 160 KB");
static_assert(kTM == 128 && kTK == 32, "a stage is 8 + 8 + TN / 16 DMAs of 1 KB: 3 or 4 per wavefront");
static_assert(kPartFloats == kTM * kTNmax, "a split-K partial slot holds one tile");
// RMSNorm sums of squares are kept per 64-column block of x
constexpr int kSsCols = 64;

enum Epi { EPI_QKV = 0, EPI_UG = 1, EPI_RESID = 2 };

// The launch's dynamic LDS, named at file scope so that every function that
// addresses it emits LDS instructions (not flat ones).
extern __shared__ __attribute__((aligned(16))) uint8_t pf_smem[];

struct PCx {
  const PParams* pp;
  int cta, grid, tid, wave, lane;
  uint32_t epoch;  // grid barriers passed
};

__device__ __forceinline__ void pf_fault(PCx& c, int code, int op, int layer, int index) {
  MK_GLOBAL Fault* f = gp(c.pp->fault);
  int32_t expect = 0;
  if (__hip_atomic_compare_exchange_strong(&f->code, &expect, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    f->cta = c.cta;
    f->pc = (int)c.epoch;
    f->op = op;
    f->step = 0;
    f->layer = layer;
    f->index = index;
  }
  stc32(c.pp->abort_flag, 1u);
}

// Grid barrier between stages: every workgroup's writes of the stage are
// released to the device (L2 written back) before it counts itself in, and
// acquired (L2 invalidated) after the count is complete.  The wait is
// bounded: past the watchdog it records a fault and raises the abort flag,
// which ends every other workgroup's wait too.  Returns true on failure.
__device__ __forceinline__ bool grid_barrier(PCx& c, int op, int layer) {
  // every wavefront's stores of the stage have reached L2 before the barrier;
  // one release then writes them back to memory for the other XCDs
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint32_t* flag = (uint32_t*)(pf_smem + kFlagOff);
  if (c.tid == 0) {
    const PParams& p = *c.pp;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(gp(p.barrier), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const uint32_t target = (c.epoch + 1) * (uint32_t)c.grid;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint32_t failed = 0;
    for (int it = 0;; ++it) {
      if (__hip_atomic_load(gp(p.barrier), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) >= target) break;
      if ((it & 15) == 15) {
        if (ldc32(p.abort_flag)) {
          failed = 1;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > p.watchdog_ticks) {
          pf_fault(c, -7, op, layer, -1);
          failed = 1;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag = failed;
    stc32(p.progress + c.cta, c.epoch + 1);
#ifndef MK_PF_STEPMARKS
    if (p.marks && c.cta == 0) *gp(p.marks + c.epoch) = __builtin_amdgcn_s_memrealtime();
#endif
  }
  __syncthreads();
  const uint32_t failed = __builtin_amdgcn_readfirstlane(*flag);
  __syncthreads();  // the flag word lies in the GEMM scales, rewritten by the next stage
  ++c.epoch;
  return failed != 0;
}

// ---------------------------------------------------------------- GEMM tiles
// One tile: rows [m0, m0 + 128) of the activations A (fp32 [rows][lda], K
// columns) times 128 weight rows (fp16, K columns each).  Wavefront w owns
// rows m0 + 32 (w % 4) .. + 32 and weight rows 64 (w / 4) .. + 64 of the
// tile: accumulator 0 the first 32 of them, accumulator 1 the next 32.  For
// paired outputs (a rotary pair of a q/k head, the gate and up rows of one
// MLP unit, two value rows) the tile's weight rows are ordered so that the
// two members of a unit land in the same lane and row of the two
// accumulators.
struct Gemm {
  int ep;                  // Epi
  int layer;
  const uint16_t* Ah;      // A operand: fp16 hi halves [rows][lda]
  const uint16_t* Al;      //            lo halves
  int lda;                 // row stride of A in halves, a multiple of 32: the K steps cover [0, lda)
  int K;                   // weight row length (A's columns K .. lda are zero)
  int norm;                // RMSNorm: output rows scaled by 1/rms(x), from p.ssp
  const uint16_t* W;       // weights: [rows][K] fp16
  int n_out;               // units (QKV, UG) or output columns (RESID)
  float* out;              // RESID: x [rows][ld_out], added to
  int ld_out;
  const uint16_t* W2;      // UG: the up rows (W holds the gate rows)
  const uint16_t* gnext;   // RESID: gain of the next RMSNorm (its x halves and sums of squares), or null
};

// Weight row (within g.W / g.W2) of tile row j of tile tn; null when j is past the matrix.
// Paired outputs: a tile's rows are groups of 64, each 32 units' first members then their
// second members.
template <int TN>
__device__ __forceinline__ const uint16_t* b_row(const PParams& p, const Gemm& g, int tn, int j) {
  const int grp = j >> 6, mem = (j >> 5) & 1, uu = j & 31;
  if (g.ep == EPI_RESID) {
    const int n = tn * TN + j;
    return n < g.n_out ? g.W + (int64_t)n * g.K : nullptr;
  }
  const int u = tn * (TN / 2) + grp * 32 + uu;
  if (u >= g.n_out) return nullptr;
  if (g.ep == EPI_UG) return (mem ? g.W2 : g.W) + (int64_t)u * g.K;
  // QKV: unit u is pair (i, i + hd/2) of head u / (hd/2) in the stacked [q; k; v] rows
  const int hh = p.hd >> 1, head = u / hh, i = u - head * hh;
  return g.W + (int64_t)(head * p.hd + i + mem * hh) * g.K;
}

// 1 KB global -> LDS transfer of one wavefront (lane i's 16 bytes at LDS
// lds_addr + 16 i), default cache policy: the operands are re-read by other tiles.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* base, uint32_t voff) {
  uint32_t save;
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  base = uniform_ptr(base);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(voff), "s"(base));
}

// Wait until at most D n of this wavefront's DMAs are in flight (D DMAs per step, n = 0 .. 3).
template <int D>
__device__ __forceinline__ void dma_wait(int n) {
  static_assert(D == 3 || D == 4, "3 or 4 DMAs per step");
  if (n >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * D) : "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * D) : "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Byte offset in a stage operand of row r's 16-byte chunk q (8 halves): the
// chunks of a 64-byte row are XOR-swizzled by (r / 4) % 4, so that the MFMA
// fragment reads of 8 consecutive lanes (8 consecutive rows) hit distinct banks.
__device__ __forceinline__ int op_chunk(int r, int q) { return r * 64 + ((q ^ ((r >> 2) & 3)) << 4); }

// One split-K item of a tile: K columns [k0, k0 + kc) of tile (tm, tn).  With
// S = 1 the item is the whole tile and applies the epilogue itself.  With S > 1
// every split stores its accumulators to its slot of p.part and counts itself
// in at the tile's counter; the split that arrives last adds the S partials in
// split order (so the result does not depend on which workgroup arrives last)
// and applies the epilogue.
//
// The operands stream through kNst LDS stages by global -> LDS DMA, kNst - 1 K
// steps ahead of the matrix cores: per step each wavefront moves 1 KB of A hi,
// A lo and B (16 rows x 64 bytes each), which the MFMAs read as they landed.
// Not inlined: its registers are allocated apart from the rest of the kernel's, so the kernel's
// spills never land in the K loop (a spill reload there is a vector load whose wait also waits for
// every DMA in flight).  It works on local copies of the context and the GEMM description.
template <int TN>
__device__ __attribute__((noinline)) void gemm_tile(PCx& c_ref, const Gemm& g_ref, int tm, int tn, int split, int S,
                                                    int tile, int tiles) {
  PCx c = c_ref;
  Gemm g = g_ref;
  // arguments arrive in vector registers: make the loop bounds and the epilogue's choices scalar
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  split = __builtin_amdgcn_readfirstlane(split);
  S = __builtin_amdgcn_readfirstlane(S);
  tile = __builtin_amdgcn_readfirstlane(tile);
  tiles = __builtin_amdgcn_readfirstlane(tiles);
  g.ep = __builtin_amdgcn_readfirstlane(g.ep);
  g.layer = __builtin_amdgcn_readfirstlane(g.layer);
  g.lda = __builtin_amdgcn_readfirstlane(g.lda);
  g.K = __builtin_amdgcn_readfirstlane(g.K);
  g.norm = __builtin_amdgcn_readfirstlane(g.norm);
  g.n_out = __builtin_amdgcn_readfirstlane(g.n_out);
  g.ld_out = __builtin_amdgcn_readfirstlane(g.ld_out);
  c.wave = __builtin_amdgcn_readfirstlane(c.wave);
  constexpr int NB = TN / 128;            // B transfers per wavefront per step
  constexpr int NJ = TN / 64;             // accumulators per wavefront: 32 weight rows each
  constexpr int kStage = stage_bytes(TN);
  constexpr int kNst = kRsOff / kStage;   // stages that fit: 4 of 32 KB (TN 256), 5 of 24 KB (TN 128)
  static_assert(kNst >= 3 && kNst - 2 <= 3, "dma_wait covers the later steps in flight");
  // the parameters as a local copy, loaded once: read through the pointer, the epilogue would reload
  // them after each of its stores, and each reload waits for the stores before it
  const PParams pcopy = *c.pp;
  const PParams& p = pcopy;
  // the values the K loop uses, as locals
  const int wave = c.wave, lane = c.lane;
  const void* const Ah = uniform_ptr(g.Ah);
  const void* const Al = uniform_ptr(g.Al);
  const void* const W = uniform_ptr(g.W);
  const int K = g.K, lda = g.lda;
  const uint32_t lds0 = (uint32_t)(uintptr_t)pf_smem;
  float* rs = (float*)(pf_smem + kRsOff);
  const int m0 = tm * kTM;
  const int kc = lda / S, k0 = split * kc;
  const int nsteps = kc / kTK;
  // DMA lanes: a transfer covers 16 rows of an operand; lane i -> row 16 j + i / 4, LDS chunk i % 4, which
  // holds the row's chunk (i % 4) ^ ((row / 4) % 4).  Wavefront w moves A hi and A lo transfer w and
  // B transfers NB w .. NB w + NB - 1.
  const int arow = 16 * wave + (lane >> 2);
  const int aq = (lane & 3) ^ ((arow >> 2) & 3);
  const uint32_t a_off = (uint32_t)((int64_t)min(m0 + arow, p.P - 1) * lda * 2) + (uint32_t)aq * 16u;
  uint32_t b_off[NB];
  int bq[NB];
#pragma unroll
  for (int h = 0; h < NB; ++h) {
    const int brow = 16 * (NB * wave + h) + (lane >> 2);
    bq[h] = (lane & 3) ^ ((brow >> 2) & 3);
    const uint16_t* br = b_row<TN>(p, g, tn, brow);
    b_off[h] = (uint32_t)((br ? br - g.W : 0) * 2);
  }
  auto issue = [&](int s) {
    const uint32_t st = lds0 + (uint32_t)((s % kNst) * kStage);
    const int k = k0 + s * kTK;
    dma16(st + wave * 1024, Ah, a_off + (uint32_t)k * 2u);
    dma16(st + kOpA + wave * 1024, Al, a_off + (uint32_t)k * 2u);
    // B rows have K columns: past K (the zero columns of A) the chunk is clamped to the row's last one
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const uint32_t kb = (uint32_t)min(k + bq[h] * 8, K - 8);
      dma16(st + 2 * kOpA + (NB * wave + h) * 1024, W, b_off[h] + kb * 2u);
    }
  };

  // wavefront (rb, cb) owns tile rows 32 rb .. + 32 and weight rows (TN / 2) cb .. + TN / 2: accumulator
  // j the 32 weight rows (TN / 2) cb + 32 j ..
  f32x16 acc[NJ] = {};
  const int rb = wave & 3, cb = wave >> 2;
  const int l32 = lane & 31, lh = lane >> 5;
  const int ar = rb * 32 + l32, br0 = cb * (TN / 2) + l32;
  auto mfma_step = [&](int s) {
    const uint8_t* st = pf_smem + (s % kNst) * kStage;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int q = sub * 2 + lh;
      const h8 ahi = *(const h8*)(st + op_chunk(ar, q));
      const h8 alo = *(const h8*)(st + kOpA + op_chunk(ar, q));
      h8 bf[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *(const h8*)(st + 2 * kOpA + op_chunk(br0 + 32 * j, q));
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bf[j], acc[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bf[j], acc[j], 0, 0, 0);
    }
  };
  // prologue: steps 0 .. kNst - 2 in flight
  for (int s = 0; s < kNst - 1 && s < nsteps; ++s) issue(s);
  // step s: wait for step s's DMAs (the later ones may stay in flight), then issue step s + kNst - 1
  // into the stage step s - 1 used, and multiply step s
  for (int s = 0; s < nsteps; ++s) {
    dma_wait<2 + NB>(min(s + kNst - 2, nsteps - 1) - s);
    __syncthreads();
    if (s + kNst - 1 < nsteps) issue(s + kNst - 1);
    mfma_step(s);
  }
  __syncthreads();  // every wavefront's MFMAs are done with the stages
  // the accumulators into LDS as the fp32 tile T[128][TN] (over the free stages), so that the split-K
  // exchange and the epilogue run as short loops over (row, column) with coalesced global accesses
  float* T = (float*)pf_smem;
  static_assert(kTM * kTNmax * 4 <= kRsOff, "the accumulator tile fits the stages");
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) T[(rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)) * TN + cb * (TN / 2) + 32 * j + l32] = acc[j][v];
  __syncthreads();
  if (S > 1) {
    float* mine = p.part + (int64_t)(split * tiles + tile) * kPartFloats;
    for (int e = c.tid * 4; e < kTM * TN; e += kPT * 4) *gp((f4*)(mine + e)) = *(const f4*)(T + e);
    // release this partial, then count it in; the last split of the tile goes on
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t* last = (uint32_t*)(pf_smem + kClaimOff + 8);
    if (c.tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t before = __hip_atomic_fetch_add(gp(p.tile_cnt + tile), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const uint32_t is_last = before == (uint32_t)S - 1;
      if (is_last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(gp(p.tile_cnt + tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);  // for the next stage
      }
      *last = is_last;
    }
    __syncthreads();
    const uint32_t is_last = __builtin_amdgcn_readfirstlane(*last);
    __syncthreads();
    if (!is_last) return;
    // the S partials in split order
    for (int e = c.tid * 4; e < kTM * TN; e += kPT * 4) {
      f4 t = {0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < S; ++sp) t += *gp((const f4*)(p.part + (int64_t)(sp * tiles + tile) * kPartFloats + e));
      *(f4*)(T + e) = t;
    }
    __syncthreads();
  }
  if (g.norm) {
    // 1 / rms of each row from its 64-column sums of squares (fixed order)
    if (c.tid < kTM) {
      const int pos = min(m0 + c.tid, p.P - 1), nblk = (p.d + kSsCols - 1) / kSsCols;
      float t = 0.f;
      for (int j = 0; j < nblk; ++j) t += *gp(p.ssp + (int64_t)j * p.P + pos);
      rs[c.tid] = 1.0f / __builtin_sqrtf(t / (float)p.d + p.eps);
    }
    __syncthreads();
  }
  // epilogue: wavefront w takes tile rows w, w + 8, ..., in groups of kEr rows whose global loads are
  // issued together (the loop would otherwise wait for each row's loads behind the previous row's stores)
  constexpr int kEr = 4;
  static_assert((kTM / kPW) % kEr == 0, "row groups");
  const int nblk = (p.d + kSsCols - 1) / kSsCols;
  if (g.ep == EPI_RESID) {
    // 64-column blocks, a column per lane: x += a, then x times the next gain as hi + lo halves and the
    // block's sum of x^2 for the next RMSNorm
    for (int b = 0; b < TN / kSsCols; ++b) {
      const int n = tn * TN + b * kSsCols + c.lane;
      const bool col = n < g.n_out;
      const int blk = (tn * TN) / kSsCols + b;
      const float gn = g.gnext && col ? (float)__builtin_bit_cast(_Float16, *gp(g.gnext + n)) : 0.f;
      for (int r0 = c.wave; r0 < kTM; r0 += kPW * kEr) {
        float x[kEr];
#pragma unroll
        for (int e = 0; e < kEr; ++e) {
          const int r = r0 + e * kPW, pos = m0 + r;
          x[e] = pos < p.P && col ? *gp(g.out + (int64_t)pos * g.ld_out + n) : 0.f;
        }
        float sq[kEr];
#pragma unroll
        for (int e = 0; e < kEr; ++e) {
          const int r = r0 + e * kPW, pos = m0 + r;
          const float sc = g.norm ? rs[r] : 1.0f;
          x[e] += T[r * TN + b * kSsCols + c.lane] * sc;
          sq[e] = x[e] * x[e];
          if (pos < p.P && col) {
            *gp(g.out + (int64_t)pos * g.ld_out + n) = x[e];
            if (g.gnext) {
              const float xg = x[e] * gn;
              const _Float16 hi = (_Float16)xg;
              *gp(p.Xh + (int64_t)pos * g.ld_out + n) = __builtin_bit_cast(uint16_t, hi);
              *gp(p.Xl + (int64_t)pos * g.ld_out + n) = __builtin_bit_cast(uint16_t, (_Float16)(xg - (float)hi));
            }
          } else {
            sq[e] = 0.f;
          }
        }
        if (g.gnext && blk < nblk) {
#pragma unroll
          for (int e = 0; e < kEr; ++e) sq[e] = wave_sum(sq[e]);
          if (c.lane == 0) {
#pragma unroll
            for (int e = 0; e < kEr; ++e) {
              const int pos = m0 + r0 + e * kPW;
              if (pos < p.P) *gp(p.ssp + (int64_t)blk * p.P + pos) = sq[e];
            }
          }
        }
      }
    }
  } else {
    // paired outputs: groups of 64 weight rows (32 units' first members, then their second members);
    // lanes 0-31 take units of an even group, lanes 32-63 of the next
    const int hh = p.hd >> 1;
    for (int gp2 = 0; gp2 < TN / 128; ++gp2) {
      const int grp = 2 * gp2 + (c.lane >> 5), uu = c.lane & 31;
      const int u = tn * (TN / 2) + grp * 32 + uu;
      if (u >= g.n_out) continue;
      // QKV: unit u is the pair (i, i + hd/2) of head u / (hd/2); q and k heads rotate it by the position's angle
      const int head = u / hh, i = u - head * hh;
      const bool rot = g.ep == EPI_QKV && head < p.nq + p.nkv;
      for (int r0 = c.wave; r0 < kTM; r0 += kPW * kEr) {
        float co[kEr], sn[kEr];
#pragma unroll
        for (int e = 0; e < kEr; ++e) {
          const int pos = min(m0 + r0 + e * kPW, p.P - 1);
          const float* cs = p.rope + ((int64_t)pos * hh + i) * 2;
          co[e] = rot ? *gp(cs) : 1.f;
          sn[e] = rot ? *gp(cs + 1) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < kEr; ++e) {
          const int r = r0 + e * kPW, pos = m0 + r;
          if (pos >= p.P) continue;
          const float sc = g.norm ? rs[r] : 1.0f;
          const float a = T[r * TN + grp * 64 + uu] * sc, b = T[r * TN + grp * 64 + 32 + uu] * sc;
          if (g.ep == EPI_UG) {
            const float m = a / (1.0f + __expf(-a)) * b;
            const _Float16 hi = (_Float16)m;
            *gp(p.Mh + (int64_t)pos * p.ldm + u) = __builtin_bit_cast(uint16_t, hi);
            *gp(p.Ml + (int64_t)pos * p.ldm + u) = __builtin_bit_cast(uint16_t, (_Float16)(m - (float)hi));
            continue;
          }
          const float ra = a * co[e] - b * sn[e], rb2 = a * sn[e] + b * co[e];
          if (head < p.nq) {
            float* qo = p.Q + (int64_t)pos * p.nq * p.hd + head * p.hd + i;
            *gp(qo) = ra;
            *gp(qo + hh) = rb2;
          } else {
            const bool isk = head < p.nq + p.nkv;
            const int kvh = head - p.nq - (isk ? 0 : p.nkv);
            uint16_t* dst = (isk ? p.kc : p.vc) + (((int64_t)g.layer * p.nkv + kvh) * p.max_seq + pos) * p.hd + i;
            *gp(dst) = __builtin_bit_cast(uint16_t, (_Float16)ra);
            *gp(dst + hh) = __builtin_bit_cast(uint16_t, (_Float16)rb2);
          }
        }
      }
    }
  }
  __syncthreads();  // the stages and scales are reused by the next tile
}

// Work distribution of a stage whose items a whole workgroup processes.
// Static: workgroup c takes items c, c + grid, ...  Dynamic (a work queue,
// "8 - Ecrire son megakernel", section 8.8): the workgroup claims its next
// item from the stage's counter while it works on the current one, so a
// workgroup that finishes early takes more items.
template <typename F>
__device__ __forceinline__ void wg_items(PCx& c, int items, F&& work) {
  const PParams& p = *c.pp;
  // one call site of `work` for both distributions (the work is inlined once)
  const bool dyn = p.dynamic != 0;
  int* slot = (int*)(pf_smem + kClaimOff);
  uint32_t* ctr = p.queue + c.epoch;
  int t = c.cta;
  if (dyn) {
    if (c.tid == 0) *slot = (int)__hip_atomic_fetch_add(gp(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    t = *slot;
    __syncthreads();
  }
  while (t < items) {
    uint32_t nxt = 0;
    if (dyn && c.tid == 0) nxt = __hip_atomic_fetch_add(gp(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    work(t);
    if (dyn) {
      if (c.tid == 0) *slot = (int)nxt;
      __syncthreads();
      t = *slot;
      __syncthreads();
    } else {
      t += c.grid;
    }
  }
}

// Split-K factor of a stage: the largest S <= 4 (a power of two) whose
// tiles x S items still fit the grid, with K a multiple of 32 S, so that a
// stage of few tiles (short prompts) still keeps every CU busy.
__device__ __forceinline__ int split_k(int tiles, int K, int grid) {
  int S = 1;
  while (S < 4 && tiles * S * 2 <= grid && K % (kTK * S * 2) == 0) S *= 2;
  return S;
}

// Order of a stage's items, for the caches: item t of the static deal runs on
// workgroup t % grid, and consecutive workgroups sit on different XCDs
// (round-robin dispatch), so t is first mapped to a position in which the
// grid / 8 workgroups of one XCD hold consecutive positions; positions then
// run down bands of kGroupM row tiles, so the 32 tiles one XCD works on at a
// time are 4 row tiles x 8 weight tiles and share their A rows and weight rows
// in that XCD's L2 (instead of every workgroup streaming the whole activation
// matrix past its own weight tile).  The split index is outermost.
constexpr int kGroupM = 4;

// A bijection of [0, items): full rounds of `grid` items are permuted within
// themselves, the last partial round keeps its order.
__device__ __forceinline__ int item_position(int t, int items, int grid, bool xcd_blocks) {
  const int r = t / grid, w = t - r * grid;
  if (!xcd_blocks || (r + 1) * grid > items) return t;
  return r * grid + (w & 7) * (grid >> 3) + (w >> 3);
}

template <int TN>
__device__ __forceinline__ void gemm_stage_tn(PCx& c, const Gemm& g) {
  const int n_tm = (c.pp->P + kTM - 1) / kTM;
  const int n_tn = g.ep == EPI_RESID ? (g.n_out + TN - 1) / TN : (g.n_out + TN / 2 - 1) / (TN / 2);
  const int tiles = n_tm * n_tn, S = split_k(tiles, g.lda, c.grid), items = tiles * S;
  const bool xcd_blocks = !c.pp->dynamic && (c.grid & 7) == 0;
  wg_items(c, items, [&](int t) {
    const int pos = item_position(t, items, c.grid, xcd_blocks);
    const int split = pos / tiles, tile = pos - split * tiles;
    // tile -> (row tile, weight tile): bands of kGroupM row tiles, column-major inside a band
    const int band = tile / (kGroupM * n_tn), first = band * kGroupM;
    const int gm = min(n_tm - first, kGroupM), in = tile - band * kGroupM * n_tn;
    const int tm = first + in % gm, tn = in / gm;
    gemm_tile<TN>(c, g, tm, tn, split, S, tm + tn * n_tm, tiles);
  });
}

// Tiles of 256 weight rows when the stage has rows enough (16 row tiles) to keep every workgroup
// busy without deep split-K, or when its 256-row tiles alone fill the grid (up/gate at 512
// tokens: 117 -> 101 us per layer): half the A traffic per output of 128-row tiles.  Other
// stages keep 128-row tiles, whose split-K partials are half the size (QKV at 512 tokens with
// 256-row tiles split 4 ways: 69 -> 92 us).
__device__ __forceinline__ void gemm_stage(PCx& c, const Gemm& g) {
  const int n_tm = (c.pp->P + kTM - 1) / kTM;
  const int rows = g.ep == EPI_RESID ? g.n_out : 2 * g.n_out;  // weight rows
  const bool wide = n_tm >= 16 || n_tm * ((rows + 255) / 256) >= c.grid;
  if (wide) gemm_stage_tn<256>(c, g);
  else gemm_stage_tn<128>(c, g);
}

// ---------------------------------------------------------------- causal attention
// Work item: query head h and a block of 16 positions.  Wavefront w takes
// positions p0 + 4 (w % 4) .. + 4 (one per 16-lane row; lane i of a row holds
// dims [i * HD/16, (i+1) * HD/16)) and the key blocks of parity w / 4; each
// keeps an online softmax in the exp2 domain (q pre-scaled by log2(e)/sqrt(hd))
// and the two key halves are merged through LDS.  Query p attends keys 0..p.
template <int HD>
__device__ __attribute__((noinline)) void att_stage(PCx& c_ref, int l) {
  // a local copy: read through the reference, its fields would be reloaded from memory (vector
  // loads that wait behind the block DMAs in flight) after every asm statement that clobbers memory
  PCx c = c_ref;
  constexpr int DL = HD / 16;          // dims per lane
  constexpr int EV = DL < 8 ? DL : 8;  // fp16 values per load
  constexpr int NV = DL / EV;          // loads per key row slice (16 bytes, or 8 for head_dim 64)
  constexpr int KB = HD >= 256 ? 4 : 8;
  const PParams& p = *c.pp;
  const int P = p.P, nqb = (P + 15) / 16, items = p.nq * nqb;
  const int row = c.lane >> 4, dl = c.lane & 15;
  const int sb = c.wave & 3, kh = c.wave >> 2;
  const float qscale = kLog2e / __builtin_sqrtf((float)HD);
  float* part = (float*)pf_smem;  // [2][16][HD + 2]
  wg_items(c, items, [&](int it) {
    const int qb = nqb - 1 - it / p.nq, h = it - (it / p.nq) * p.nq;
    const int g = h * p.nkv / p.nq;
    const int p0 = qb * 16, qi = sb * 4 + row, pq = p0 + qi;
    const bool qok = pq < P;
    const int kmax = min(p0 + 15, P - 1);
    const int lim = qok ? pq : kmax;  // last key this lane's query attends
    float q[DL], o[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      q[e] = qok ? *gp(p.Q + (int64_t)pq * p.nq * HD + h * HD + dl * DL + e) * qscale : 0.f;
      o[e] = 0.f;
    }
    float m = -INFINITY, ls = 0.f;
    const int64_t hoff = ((int64_t)l * p.nkv + g) * p.max_seq * HD + dl * DL;
    const uint16_t* kb = p.kc + hoff;
    const uint16_t* vb = p.vc + hoff;
    const int nblk = kmax / KB + 1;
    for (int b = kh; b < nblk; b += 2) {
      const int t0 = b * KB;
      u4 kr[KB][NV], vr[KB][NV];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int t = t0 + j;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          kr[j][v] = u4{0u, 0u, 0u, 0u};
          vr[j][v] = u4{0u, 0u, 0u, 0u};
          if (t <= kmax) {
            const int64_t o = (int64_t)t * HD + v * EV;
            if constexpr (EV == 8) {
              kr[j][v] = *gp((const u4*)(kb + o));
              vr[j][v] = *gp((const u4*)(vb + o));
            } else {
              const u2 k2 = *gp((const u2*)(kb + o)), v2 = *gp((const u2*)(vb + o));
              kr[j][v] = u4{k2[0], k2[1], 0u, 0u};
              vr[j][v] = u4{v2[0], v2[1], 0u, 0u};
            }
          }
        }
      }
      float s[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const h8 kh8 = __builtin_bit_cast(h8, kr[j][v]);
#pragma unroll
          for (int e = 0; e < EV; ++e) acc = fmaf(q[v * EV + e], (float)kh8[e], acc);
        }
        s[j] = acc;
      }
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        float v = s[j];
        v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
        v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
        v += dpp<0x141>(v);  // row_half_mirror
        v += dpp<0x140>(v);  // row_mirror: the 16-lane row sum in every lane of the row
        s[j] = t0 + j <= lim ? v : -INFINITY;
      }
      float mb = m;
#pragma unroll
      for (int j = 0; j < KB; ++j) mb = fmaxf(mb, s[j]);
      const float al = mb == -INFINITY ? 1.f : exp2f(m - mb);
      ls *= al;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] *= al;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const float w = s[j] == -INFINITY ? 0.f : exp2f(s[j] - mb);
        ls += w;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const h8 vh = __builtin_bit_cast(h8, vr[j][v]);
#pragma unroll
          for (int e = 0; e < EV; ++e) o[v * EV + e] = fmaf(w, (float)vh[e], o[v * EV + e]);
        }
      }
      m = mb;
    }
    // merge the two key halves: partials [kh][query][m, l, o[HD]]
    float* rec = part + (kh * 16 + qi) * (HD + 2);
    if (dl == 0) {
      rec[0] = m;
      rec[1] = ls;
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) rec[2 + dl * DL + e] = o[e];
    __syncthreads();
    for (int i = c.tid; i < 16 * HD; i += kPT) {
      const int q2 = i / HD, dd = i - q2 * HD, pos = p0 + q2;
      if (pos >= P) continue;
      const float* r0 = part + q2 * (HD + 2);
      const float* r1 = part + (16 + q2) * (HD + 2);
      const float M = fmaxf(r0[0], r1[0]);
      const float a0 = r0[0] == -INFINITY ? 0.f : exp2f(r0[0] - M);
      const float a1 = r1[0] == -INFINITY ? 0.f : exp2f(r1[0] - M);
      const float ov = (a0 * r0[2 + dd] + a1 * r1[2 + dd]) / (a0 * r0[1] + a1 * r1[1]);
      const _Float16 hi = (_Float16)ov;
      const int64_t oi = (int64_t)pos * p.ldo + h * HD + dd;
      *gp(p.Oh + oi) = __builtin_bit_cast(uint16_t, hi);
      *gp(p.Ol + oi) = __builtin_bit_cast(uint16_t, (_Float16)(ov - (float)hi));
    }
    __syncthreads();
  });
}

// ---------------------------------------------------------------- causal attention on MFMA
// Work item of one wavefront: query head h and 32 consecutive positions.  It
// walks the keys 0 .. (last query) in blocks of 32 with an online softmax in
// the exp2 domain (q pre-scaled by log2(e)/sqrt(hd)):
//   S^T = K Q^T    A = the K block (rows = keys, K-dim = head dims), loaded
//                  straight from the cache; B = Q^T as fp16 hi + lo halves
//   O^T += V^T P^T A = the V block transposed through this wavefront's LDS
//                  slice; B = the probabilities P^T as fp16 hi + lo halves
// With the products transposed this way, lane l owns query l % 32 in every
// accumulator (S^T columns, O^T columns), so the softmax statistics and the
// rescaling of O stay in the lane; the other 16 keys of a block sit in lane
// l ^ 32.  The probabilities enter the second product in the order the S^T
// accumulator holds them, and the V^T operand reads its keys in that order.
constexpr int kVtStride = 40;  // halves per V^T row in LDS (32 keys + padding)
static_assert(kPW * 128 * kVtStride * 2 <= kClaimOff && 2 * 16 * (256 + 2) * 4 <= kClaimOff, "claim slot overlaps attention LDS");

template <int HD>
__device__ __attribute__((noinline)) void att_stage_mfma(PCx& c_ref, int l) {
  // a local copy: read through the reference, its fields would be reloaded from memory (vector
  // loads that wait behind the block DMAs in flight) after every asm statement that clobbers memory
  PCx c = c_ref;
  constexpr int KS = HD / 16;  // MFMA K-steps over the head dims
  constexpr int DB = HD / 32;  // 32-dim blocks of O^T
  const PParams& p = *c.pp;
  // the fields the item loop uses, as locals: p is read through a pointer, and every asm statement
  // that clobbers memory would make the compiler reload them (loads that wait behind the DMAs)
  uint16_t* const Ohp = (uint16_t*)uniform_ptr(p.Oh);
  uint16_t* const Olp = (uint16_t*)uniform_ptr(p.Ol);
  const float* const Qp = (const float*)uniform_ptr(p.Q);
  const int ldo = p.ldo, nq = p.nq, nkv = p.nkv, max_seq = p.max_seq;
  const int P = p.P, nqb = (P + 31) / 32, items = nq * nqb;
  const int i32 = c.lane & 31, hh = c.lane >> 5;
  const float qscale = kLog2e / __builtin_sqrtf((float)HD);
  _Float16* vt = (_Float16*)pf_smem + c.wave * HD * kVtStride;  // this wavefront's V^T block [HD][kVtStride]
  const int nw = c.grid * kPW, gw = c.cta * kPW + c.wave;
  // static: wavefront gw takes items gw, gw + nw, ...; dynamic: each wavefront claims its next
  // item from the stage's counter while it works on the current one
  uint32_t* ctr = p.queue + c.epoch;
  auto claim = [&]() -> int {
    uint32_t v = 0;
    if (c.lane == 0) v = __hip_atomic_fetch_add(gp(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return v;
  };
  int it = p.dynamic ? __builtin_amdgcn_readfirstlane(claim()) : gw;
  while (it < items) {
    const int nxt_raw = p.dynamic ? claim() : it + nw;
    // the longest items (latest query blocks) first
    const int qb = nqb - 1 - it / nq, h = it - (it / nq) * nq;
    const int g = h * nkv / nq;
    const int q0 = qb * 32, pq = q0 + i32;           // this lane's query
    const int lim = min(pq, P - 1);                  // last key it attends
    const int kmax = min(q0 + 31, P - 1);            // last key of any query of the block
    // Q^T operands: dims 16 s + 8 hh + e of query pq, as hi and lo halves
    h8 qh[KS], ql[KS];
    {
      const float* qrow = Qp + (int64_t)min(pq, P - 1) * nq * HD + h * HD + 8 * hh;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const f4 a = *gp((const f4*)(qrow + 16 * s)), b = *gp((const f4*)(qrow + 16 * s + 4));
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = v[e] * qscale;
          qh[s][e] = (_Float16)x;
          ql[s][e] = (_Float16)(x - (float)qh[s][e]);
        }
      }
    }
    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x16{};
    float m = -INFINITY, ls = 0.f;
    const int64_t hbase = ((int64_t)l * nkv + g) * max_seq * HD;
    const uint16_t* kbase = p.kc + hbase;
    const uint16_t* vbase = p.vc + hbase;
    for (int kb0 = 0; kb0 <= kmax; kb0 += 32) {
      // S^T block: lane l holds query pq and keys kb0 + 8 (v / 4) + 4 hh + v % 4
      const int key = kb0 + i32;                      // this lane's K / V row for the operands
      const bool kin = key <= kmax;
      f32x16 st = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u4 kr = kin ? *gp((const u4*)(kbase + (int64_t)key * HD + 16 * s + 8 * hh)) : u4{0u, 0u, 0u, 0u};
        const h8 ka = __builtin_bit_cast(h8, kr);
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qh[s], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, ql[s], st, 0, 0, 0);
      }
      // V block -> V^T in LDS: lane (key i32, half hh) writes dims [HD/2 hh, HD/2 (hh + 1)) of its key
#pragma unroll
      for (int v8 = 0; v8 < HD / 16; ++v8) {
        const int d0 = hh * (HD / 2) + v8 * 8;
        const u4 vr = kin ? *gp((const u4*)(vbase + (int64_t)key * HD + d0)) : u4{0u, 0u, 0u, 0u};
        const h8 vh = __builtin_bit_cast(h8, vr);
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(d0 + e) * kVtStride + i32] = vh[e];
      }
      // mask, block maximum (this lane's 16 keys, then the other 16 in lane l ^ 32)
      float mb = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = kb0 + (v >> 2) * 8 + hh * 4 + (v & 3);
        st[v] = kk <= lim ? st[v] : -INFINITY;
        mb = fmaxf(mb, st[v]);
      }
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float mn = fmaxf(m, mb);
      const float al = mn == -INFINITY ? 1.f : exp2f(m - mn);
      ls *= al;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= al;
      m = mn;
      // probabilities, as the B operand of O^T += V^T P^T in two K-steps of 16 keys
      h8 ph[2], pl[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float w = st[v] == -INFINITY ? 0.f : exp2f(st[v] - mn);
        ls += w;
        const _Float16 hi = (_Float16)w;
        ph[v >> 3][v & 7] = hi;
        pl[v >> 3][v & 7] = (_Float16)(w - (float)hi);
      }
      // V^T operand of step t: dim 32 b + i32, keys 16 t + 4 hh + {0..3} and 16 t + 8 + 4 hh + {0..3}
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const _Float16* row = vt + (b * 32 + i32) * kVtStride;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          const h4 x0 = *(const h4*)(row + 16 * t + 4 * hh);
          const h4 x1 = *(const h4*)(row + 16 * t + 8 + 4 * hh);
          const h8 va = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, ph[t], o[b], 0, 0, 0);
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pl[t], o[b], 0, 0, 0);
        }
      }
    }
    // the query's sum over all keys: this lane's keys plus those of lane l ^ 32
    const float lt = ls + __shfl_xor(ls, 32);
    if (pq < P) {
      const int64_t orow = (int64_t)pq * ldo + h * HD;
      const float inv = 1.0f / lt;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          // dims 32 b + 8 a + 4 hh + {0..3}: registers 4 a .. 4 a + 3, as fp16 hi and lo halves
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          h4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = o[b][4 * a + e] * inv;
            hi[e] = (_Float16)v;
            lo[e] = (_Float16)(v - (float)hi[e]);
          }
          const int64_t oi = orow + 32 * b + 8 * a + 4 * hh;
          *gp((u2*)(Ohp + oi)) = __builtin_bit_cast(u2, hi);
          *gp((u2*)(Olp + oi)) = __builtin_bit_cast(u2, lo);
        }
    }
    it = p.dynamic ? __builtin_amdgcn_readfirstlane(nxt_raw) : nxt_raw;
  }
}

// ---------------------------------------------------------------- causal attention, workgroup-cooperative
// Work item of a workgroup: kv head g and a super-block of 32 QPW consecutive
// queries, QPW = 8 / G for G query heads per kv head; wavefront w takes query
// head g G + w / QPW and the 32 queries (w % QPW) of the super-block.  All 8
// wavefronts walk the same key blocks of 32, which the workgroup stages once:
// the K and V blocks by global -> LDS DMA kAttNst - 1 blocks ahead (each row's
// 16-byte chunks XOR-swizzled by the row, so that 8 consecutive key rows read
// at one dim hit distinct banks), V transposed to V^T once per block by all
// threads.  Per block, every wavefront whose queries reach it computes
// S^T = K Q^T and O^T += V^T P^T as the per-wavefront version does (lane l
// owns query l % 32; online softmax in the exp2 domain).
constexpr int kAttNst = 3;

// KSPLIT: the key-chunk variant for prompts with fewer items than workgroups (a template parameter,
// so that the long prompts' variant carries none of the chunk bookkeeping in its registers).
template <int HD, bool KSPLIT>
__device__ __attribute__((noinline)) void att_stage_wg(PCx& c_ref, int l) {
  // a local copy: read through the reference, its fields would be reloaded from memory (vector
  // loads that wait behind the block DMAs in flight) after every asm statement that clobbers memory
  PCx c = c_ref;
  constexpr int KS = HD / 16;              // MFMA K-steps over the head dims
  constexpr int DB = HD / 32;              // 32-dim blocks of O^T
  constexpr int CPR = HD / 8;              // 16-byte chunks per K / V row
  constexpr int BLK = 32 * HD * 2;         // bytes of a K or V block of 32 keys
  constexpr int TPB = 2 * BLK / 1024;      // 1 KB transfers per block (K and V)
  constexpr int DPW = TPB / kPW;           // transfers per wavefront per block
  constexpr int RPT = 1024 / (HD * 2);     // key rows per transfer
  static_assert(DPW * kPW == TPB && DPW >= 1 && DPW <= 2, "K and V blocks split evenly over the wavefronts");
  static_assert(kAttNst * 2 * BLK + 2 * HD * kVtStride * 2 <= kClaimOff, "attention staging overlaps the claim slot");
  const PParams& p = *c.pp;
  // the fields the item loop uses, as locals: p is read through a pointer, and every asm statement
  // that clobbers memory would make the compiler reload them (loads that wait behind the DMAs)
  uint16_t* const Ohp = (uint16_t*)uniform_ptr(p.Oh);
  uint16_t* const Olp = (uint16_t*)uniform_ptr(p.Ol);
  const float* const Qp = (const float*)uniform_ptr(p.Q);
  const int ldo = p.ldo, nq = p.nq, nkv = p.nkv, max_seq = p.max_seq;
  const int G = nq / nkv, QPW = kPW / G, SB = 32 * QPW;
  const int P = p.P, nsb = (P + SB - 1) / SB;
  // key blocks of super-block sbi's queries (causal: up to its last query)
  auto nblk_of = [&](int sbi) { return min(sbi * SB + SB - 1, P - 1) / 32 + 1; };
  // Short prompts have fewer (kv head, super-block) items than workgroups, and the latest
  // super-block's item alone takes as long as the whole stage.  Then each item's keys are split
  // into chunks of CB blocks, so that the chunks about fill the grid; a chunk writes its unnormalised
  // partial (m, l, O) and the last chunk of an item to finish merges them in chunk order.
  int CB = 1 << 30;
  if (KSPLIT) {
    int total = 0;
    for (int sbi = 0; sbi < nsb; ++sbi) total += nblk_of(sbi);
    CB = max(4, (nkv * total + c.grid - 1) / c.grid);
  }
  int items = 0;
  for (int sbi = 0; sbi < nsb; ++sbi) items += nkv * ((nblk_of(sbi) + CB - 1) / CB);
  const int i32 = c.lane & 31, hh = c.lane >> 5;
  const float qscale = kLog2e / __builtin_sqrtf((float)HD);
  const uint32_t lds0 = (uint32_t)(uintptr_t)pf_smem;
  _Float16* vt_base = (_Float16*)(pf_smem + kAttNst * 2 * BLK);  // [2][HD][kVtStride]
  // static deal in rounds of `grid` items: every other round takes its super-blocks in reverse, so a
  // workgroup that drew one of the longest items in one round draws one of the shortest in the next
  // (with grid a multiple of n_kv the kv head of a workgroup's items stays the same)
  const bool snake = !KSPLIT && !p.dynamic && c.grid % nkv == 0;
  wg_items(c, items, [&](int it) {
    if (snake && (it / c.grid) % 2 == 1) {
      const int r0 = it - it % c.grid, j = it - r0, nr = min(c.grid, items - r0);
      it = r0 + (nr / nkv - 1 - j / nkv) * nkv + j % nkv;
    }
    // the longest items (latest query super-blocks) first; per super-block its key chunks, then the
    // kv heads (one chunk per item unless the keys are split)
    int sbi = nsb - 1, base = 0, nch = (nblk_of(sbi) + CB - 1) / CB;
    while (it - base >= nch * nkv) {
      base += nch * nkv;
      --sbi;
      nch = (nblk_of(sbi) + CB - 1) / CB;
    }
    const int chunk = (it - base) / nkv, g = (it - base) - chunk * nkv;
    const int h = g * G + c.wave / QPW;
    const int q0 = sbi * SB + (c.wave % QPW) * 32, pq = q0 + i32;
    const bool active = q0 < P;
    const int lim = min(pq, P - 1);                    // last key this lane's query attends
    const int kmax_w = min(q0 + 31, P - 1);            // last key of this wavefront's queries
    const int kmax = min(sbi * SB + SB - 1, P - 1);    // last key of the workgroup's queries
    const int b0 = chunk * min(CB, kmax / 32 + 1), b1 = min(kmax / 32 + 1, b0 + CB);  // this item's key blocks
    // Q^T operands: dims 16 s + 8 hh + e of query pq, as hi and lo halves
    h8 qh[KS], ql[KS];
    {
      const float* qrow = Qp + (int64_t)min(pq, P - 1) * nq * HD + h * HD + 8 * hh;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const f4 a = *gp((const f4*)(qrow + 16 * s)), b = *gp((const f4*)(qrow + 16 * s + 4));
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = v[e] * qscale;
          qh[s][e] = (_Float16)x;
          ql[s][e] = (_Float16)(x - (float)qh[s][e]);
        }
      }
    }
    // DMA lanes: transfer j of a block (K: j < TPB / 2, V: the rest) covers key rows RPT (j % (TPB / 2)) ..;
    // lane i -> row rr = that + i / CPR, LDS chunk i % CPR, which holds the row's chunk (i % CPR) ^ (rr % CPR)
    const int64_t head_row = ((int64_t)l * nkv + g) * max_seq;
    const void* const kcp = uniform_ptr(p.kc);
    const void* const vcp = uniform_ptr(p.vc);
    auto issue = [&](int b) {
      const uint32_t st = lds0 + (uint32_t)((b % kAttNst) * 2 * BLK);
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int j = c.wave * DPW + d, isv = j >= TPB / 2, jj = isv ? j - TPB / 2 : j;
        const int rr = jj * RPT + c.lane / CPR, cc = c.lane % CPR, gq = cc ^ (rr % CPR);
        const int key = min(b * 32 + rr, kmax);  // rows past the last key repeat it: finite, and masked
        const uint32_t voff = (uint32_t)((head_row + key) * HD * 2) + (uint32_t)gq * 16u;
        dma16(st + isv * BLK + jj * 1024, isv ? vcp : kcp, voff);
      }
    };
    auto wait_block = [&](int later) {  // later blocks of DMAs that may stay in flight (0 or 1)
      const int n = later * DPW;
      if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x16{};
    float m = -INFINITY, ls = 0.f;
    for (int b = b0; b < b0 + kAttNst - 1 && b < b1; ++b) issue(b);
    for (int b = b0; b < b1; ++b) {
      wait_block(min(b + kAttNst - 2, b1 - 1) - b);
      __syncthreads();  // block b landed (every wavefront's DMAs); block b - 1's stage and V^T b - 2 are free
      if (b + kAttNst - 1 < b1) issue(b + kAttNst - 1);
      const uint8_t* kst = pf_smem + (b % kAttNst) * 2 * BLK;
      _Float16* vt = vt_base + (b & 1) * HD * kVtStride;
      // V block -> V^T: thread t takes key t % 32, dims 8 (t / 32) .. + 8, so the lanes of a 2-byte
      // store write consecutive keys of one V^T row (keys split over the lanes instead hit the same
      // LDS banks 8-16 ways: the V^T rows sit 80 bytes apart)
      if (c.tid < 32 * CPR) {
        const int rr = c.tid % 32, gq = c.tid / 32;
        const h8 vh = *(const h8*)(kst + BLK + rr * HD * 2 + ((gq ^ (rr % CPR)) << 4));
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(gq * 8 + e) * kVtStride + rr] = vh[e];
      }
      __syncthreads();
      const int kb0 = b * 32;
      if (!active || kb0 > kmax_w) continue;  // no query of this wavefront reaches the block
      // S^T block: lane l holds query pq and keys kb0 + 8 (v / 4) + 4 hh + v % 4
      f32x16 st = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int gq = 2 * s + hh;
        const h8 ka = *(const h8*)(kst + i32 * HD * 2 + ((gq ^ (i32 % CPR)) << 4));
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qh[s], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, ql[s], st, 0, 0, 0);
      }
      float mb = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = kb0 + (v >> 2) * 8 + hh * 4 + (v & 3);
        st[v] = kk <= lim ? st[v] : -INFINITY;
        mb = fmaxf(mb, st[v]);
      }
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float mn = fmaxf(m, mb);
      const float al = mn == -INFINITY ? 1.f : exp2f(m - mn);
      ls *= al;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] *= al;
      m = mn;
      h8 ph[2], pl[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float w = st[v] == -INFINITY ? 0.f : exp2f(st[v] - mn);
        ls += w;
        const _Float16 hi = (_Float16)w;
        ph[v >> 3][v & 7] = hi;
        pl[v >> 3][v & 7] = (_Float16)(w - (float)hi);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const _Float16* row = vt + (d * 32 + i32) * kVtStride;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          const h4 x0 = *(const h4*)(row + 16 * t + 4 * hh);
          const h4 x1 = *(const h4*)(row + 16 * t + 8 + 4 * hh);
          const h8 va = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, ph[t], o[d], 0, 0, 0);
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pl[t], o[d], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next item's DMAs reuse the stages
    float lt = ls + __shfl_xor(ls, 32);
    if (KSPLIT && nch > 1) {
      // this chunk's partial: [item][wavefront][field][lane], fields m, l, then O^T's accumulators
      // (items < 2 grid: the chunks are sized to about fill the grid, plus one partial chunk per
      // (kv head, super-block), of which there are fewer than the grid)
      constexpr int NF = 2 + DB * 16;
      static_assert(kPW * NF * 64 <= kAttPartFloats, "a chunk's partial fits its slot");
      float* const part = p.part;
      float* mine = part + (int64_t)it * kAttPartFloats + (int64_t)c.wave * NF * 64 + c.lane;
      *gp(mine) = m;
      *gp(mine + 64) = lt;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) *gp(mine + (2 + d * 16 + v) * 64) = o[d][v];
      // release it and count it in; the last chunk of the item merges
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      uint32_t* last = (uint32_t*)(pf_smem + kClaimOff + 8);
      uint32_t* const cnt = p.tile_cnt + sbi * nkv + g;
      if (c.tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t before = __hip_atomic_fetch_add(gp(cnt), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        const uint32_t is_last = before == (uint32_t)nch - 1;
        if (is_last) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          __hip_atomic_store(gp(cnt), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);  // for the next layer
        }
        *last = is_last;
      }
      __syncthreads();
      const uint32_t is_last = __builtin_amdgcn_readfirstlane(*last);
      __syncthreads();
      if (!is_last) return;
      // merge the item's chunks in chunk order: M = max m, L = sum 2^(m - M) l, O = sum 2^(m - M) O
      const int first = base + g;  // chunk k of the item is item first + k nkv
      float M = -INFINITY;
      for (int k = 0; k < nch; ++k) M = fmaxf(M, *gp(part + (int64_t)(first + k * nkv) * kAttPartFloats + (int64_t)c.wave * NF * 64 + c.lane));
      lt = 0.f;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = f32x16{};
      for (int k = 0; k < nch; ++k) {
        const float* src = part + (int64_t)(first + k * nkv) * kAttPartFloats + (int64_t)c.wave * NF * 64 + c.lane;
        const float mk = *gp(src);
        const float wk = mk == -INFINITY ? 0.f : exp2f(mk - M);
        lt += wk * *gp(src + 64);
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[d][v] += wk * *gp(src + (2 + d * 16 + v) * 64);
      }
    }
    if (active && pq < P) {
      const int64_t orow = (int64_t)pq * ldo + h * HD;
      const float inv = 1.0f / lt;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          h4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = o[d][4 * a + e] * inv;
            hi[e] = (_Float16)v;
            lo[e] = (_Float16)(v - (float)hi[e]);
          }
          const int64_t oi = orow + 32 * d + 8 * a + 4 * hh;
          *gp((u2*)(Ohp + oi)) = __builtin_bit_cast(u2, hi);
          *gp((u2*)(Olp + oi)) = __builtin_bit_cast(u2, lo);
        }
    }
  });
}

}  // namespace

__global__ __launch_bounds__(kPT, 1) void mk_prefill_kernel(const PParams* __restrict__ ppp) {
  const PParams& p = *ppp;
  PCx c;
  c.pp = ppp;
  c.cta = blockIdx.x;
  c.grid = gridDim.x;
  c.tid = threadIdx.x;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.epoch = 0;
  // the residual stream starts as the embedding rows of the prompt; with it, x times layer 0's
  // first gain as fp16 hi + lo halves and x^2 summed over each 64-column block (one wavefront
  // per (position, block), a column per lane)
  {
    const int nblk = (p.d + kSsCols - 1) / kSsCols, items = p.P * nblk;
    const uint16_t* g1 = p.norms;
    for (int it = c.cta * kPW + c.wave; it < items; it += c.grid * kPW) {
      const int pos = it / nblk, blk = it - pos * nblk;
      const uint16_t* erow = p.embed + (int64_t)*gp(p.ids + pos) * p.d;
      float sq = 0.f;
      {
        const int k = blk * kSsCols + c.lane;
        if (k < p.d) {
          const float x = (float)__builtin_bit_cast(_Float16, *gp(erow + k));
          const int64_t i = (int64_t)pos * p.d + k;
          *gp(p.X + i) = x;
          const float xg = x * (float)__builtin_bit_cast(_Float16, *gp(g1 + k));
          const _Float16 hi = (_Float16)xg;
          *gp(p.Xh + i) = __builtin_bit_cast(uint16_t, hi);
          *gp(p.Xl + i) = __builtin_bit_cast(uint16_t, (_Float16)(xg - (float)hi));
          sq = fmaf(x, x, sq);
        }
      }
      sq = wave_sum(sq);
      if (c.lane == 0) *gp(p.ssp + (int64_t)blk * p.P + pos) = sq;
    }
  }
  if (grid_barrier(c, OP_QKV, 0)) return;
  const int qd = p.nq * p.hd, kvd = p.nkv * p.hd;
  const int64_t per_layer = (int64_t)(qd + 2 * kvd) * p.d + (int64_t)p.d * qd + 3LL * p.f * p.d;
  const int G = p.nq / p.nkv;
  const bool wg_att = G == 1 || G == 2 || G == 4 || G == 8;  // query heads of a kv head split the 8 wavefronts
  // fewer (kv head, super-block) attention items than workgroups: split their keys into chunks
  const bool ksplit = wg_att && p.nkv * ((p.P + 32 * (kPW / G) - 1) / (32 * (kPW / G))) < c.grid;
  // 5 stages per layer; every GEMM runs from one call site (its code is in the kernel once)
  for (int st = 0; st < 5 * p.L; ++st) {
    const int l = st / 5, kind = st - 5 * l;
    const uint16_t* wl = p.canon + l * per_layer;
    const uint16_t* wo = wl + (int64_t)(qd + 2 * kvd) * p.d;
    const uint16_t* wg = wo + (int64_t)p.d * qd;
    const uint16_t* wu = wg + (int64_t)p.f * p.d;
    const uint16_t* wd = wu + (int64_t)p.f * p.d;
    const uint16_t* g2 = p.norms + ((int64_t)l * 2 + 1) * p.d;
    // the next layer's first gain (none after the last layer: its x feeds no GEMM here)
    const uint16_t* gn = l + 1 < p.L ? p.norms + (int64_t)(l + 1) * 2 * p.d : nullptr;
    if (kind == 1) {
      if (p.hd == 64) {
        if (wg_att && ksplit) att_stage_wg<64, true>(c, l);
        else if (wg_att) att_stage_wg<64, false>(c, l);
        else att_stage_mfma<64>(c, l);
      } else if (p.hd == 128) {
        if (wg_att && ksplit) att_stage_wg<128, true>(c, l);
        else if (wg_att) att_stage_wg<128, false>(c, l);
        else att_stage_mfma<128>(c, l);
      } else {
        att_stage<256>(c, l);
      }
    } else {
      Gemm g;
      if (kind == 0)
        g = Gemm{EPI_QKV, l, p.Xh, p.Xl, p.d, p.d, 1, wl, (p.nq + 2 * p.nkv) * (p.hd / 2), nullptr, 0, nullptr, nullptr};
      else if (kind == 2)
        g = Gemm{EPI_RESID, l, p.Oh, p.Ol, p.ldo, qd, 0, wo, p.d, p.X, p.d, nullptr, g2};
      else if (kind == 3)
        g = Gemm{EPI_UG, l, p.Xh, p.Xl, p.d, p.d, 1, wg, p.f, nullptr, 0, wu, nullptr};
      else
        g = Gemm{EPI_RESID, l, p.Mh, p.Ml, p.ldm, p.f, 0, wd, p.d, p.X, p.d, nullptr, gn};
      gemm_stage(c, g);
    }
    const int op = kind == 0 ? OP_QKV : kind == 1 ? OP_ATT : kind == 2 ? OP_OPROJ : kind == 3 ? OP_UPGATE : OP_DOWN;
    if (grid_barrier(c, op, l)) return;
  }
}

// ---------------------------------------------------------------- host-side wrappers (internal)
#define MK_INTERNAL __attribute__((visibility("hidden")))
extern "C" {
// LDS bytes of the prefill kernel for head_dim hd: the GEMM staging or the
// attention merge, whichever is larger.
MK_INTERNAL int mk_prefill_lds_bytes(int hd) {
  // every stage's use (GEMM staging; head_dim 256: the merge of the vector-unit attention;
  // 64 and 128: one V^T block per wavefront) lies below the work-queue slot
  (void)hd;
  return kClaimOff + 16;
}
MK_INTERNAL hipError_t mk_prefill_attributes(int lds_bytes, int* occupancy) {
  hipError_t e = hipFuncSetAttribute((const void*)mk_prefill_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, mk_prefill_kernel, kPT, lds_bytes);
}
MK_INTERNAL hipError_t mk_launch_prefill(const PParams* pp_dev, int grid, int lds_bytes, hipStream_t s) {
  hipLaunchKernelGGL(mk_prefill_kernel, dim3(grid), dim3(kPT), lds_bytes, s, pp_dev);
  return hipGetLastError();
}
}
