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
constexpr int kTN = 128;               // GEMM tile: weight rows (64 units of two rows, or 128 columns)
constexpr int kTK = 32;                // K per pipeline step (two MFMA steps of 16)
constexpr int kLS = kTK + 8;           // LDS row stride in halves (padding spreads the banks)
constexpr int kOpHalves = kTM * kLS;   // one staged operand tile
// LDS: A hi, A lo, B, each double-buffered, then the row scales
constexpr int kGemmLdsBytes = 6 * kOpHalves * 2 + kTM * 4;
// The work-queue slot a workgroup reads its claimed tile from, past every
// stage's own LDS use (the largest: 8 wavefronts' V^T blocks at head_dim 128).
constexpr int kClaimOff = 8 * 128 * 40 * 2;
static_assert(kClaimOff >= kGemmLdsBytes, "claim slot overlaps the GEMM staging");

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
  uint32_t* flag = (uint32_t*)(pf_smem + kGemmLdsBytes - 4);
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
    if (p.marks && c.cta == 0) *gp(p.marks + c.epoch) = __builtin_amdgcn_s_memrealtime();
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
  const float* A;          // activations
  int lda, K;              // row stride and columns of A (= weight row length)
  const uint16_t* gain;    // RMSNorm gain (fp16 [K]) or null: no norm
  const uint16_t* W;       // weights: [rows][K] fp16
  int n_out;               // units (QKV, UG) or output columns (RESID)
  float* out;              // RESID: x [rows][ld_out], added to; UG: m [rows][ld_out]
  int ld_out;
  const uint16_t* W2;      // UG: the up rows (W holds the gate rows)
};

// Weight row (within g.W / g.W2) of tile row j of tile tn; null when j is past the matrix.
__device__ __forceinline__ const uint16_t* b_row(const PParams& p, const Gemm& g, int tn, int j) {
  const int cb = j >> 6, mem = (j >> 5) & 1, uu = j & 31;
  if (g.ep == EPI_RESID) {
    const int n = tn * kTN + j;
    return n < g.n_out ? g.W + (int64_t)n * g.K : nullptr;
  }
  const int u = tn * 64 + cb * 32 + uu;
  if (u >= g.n_out) return nullptr;
  if (g.ep == EPI_UG) return (mem ? g.W2 : g.W) + (int64_t)u * g.K;
  // QKV: unit u is pair (i, i + hd/2) of head u / (hd/2) in the stacked [q; k; v] rows
  const int hh = p.hd >> 1, head = u / hh, i = u - head * hh;
  return g.W + (int64_t)(head * p.hd + i + mem * hh) * g.K;
}

__device__ __forceinline__ void gemm_tile(PCx& c, const Gemm& g, int tm, int tn) {
  const PParams& p = *c.pp;
  _Float16* Ahi = (_Float16*)pf_smem;
  _Float16* Alo = Ahi + 2 * kOpHalves;
  _Float16* Bt = Alo + 2 * kOpHalves;
  float* rs = (float*)(Bt + 2 * kOpHalves);
  const int m0 = tm * kTM;
  // staging: thread t loads row t / 4, columns (t % 4) * 8 .. + 8 of the K step (A and B alike)
  const int srow = c.tid >> 2, skq = (c.tid & 3) * 8;
  const bool arow_ok = m0 + srow < p.P;
  const float* arow = g.A + (int64_t)(m0 + srow) * g.lda;
  const uint16_t* brow = b_row(p, g, tn, srow);
  const int nsteps = (g.K + kTK - 1) / kTK;
  float ss = 0.f;
  f4 av0, av1;
  u4 bv, gv;

  auto load = [&](int s) {
    const int k = s * kTK + skq;
    const bool kin = k < g.K;  // K is a multiple of 8: an 8-group is wholly in or out
    if (arow_ok && kin) {
      av0 = *gp((const f4*)(arow + k));
      av1 = *gp((const f4*)(arow + k + 4));
    } else {
      av0 = f4{0.f, 0.f, 0.f, 0.f};
      av1 = av0;
    }
    bv = (brow && kin) ? *gp((const u4*)(brow + k)) : u4{0u, 0u, 0u, 0u};
    if (g.gain) gv = kin ? *gp((const u4*)(g.gain + k)) : u4{0u, 0u, 0u, 0u};
  };
  auto stage = [&](int buf) {
    float a[8] = {av0[0], av0[1], av0[2], av0[3], av1[0], av1[1], av1[2], av1[3]};
    h8 hi, lo;
    if (g.gain) {
      const h8 gh = __builtin_bit_cast(h8, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(a[e], a[e], ss);
        a[e] *= (float)gh[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (_Float16)a[e];
      lo[e] = (_Float16)(a[e] - (float)hi[e]);
    }
    const int o = buf * kOpHalves + srow * kLS + skq;
    *(h8*)(Ahi + o) = hi;
    *(h8*)(Alo + o) = lo;
    *(u4*)(Bt + o) = bv;
  };

  f32x16 acc0 = {}, acc1 = {};
  const int rb = c.wave & 3, cb = c.wave >> 2;
  const int l32 = c.lane & 31, lh = c.lane >> 5;
  load(0);
  stage(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load(s + 1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ko = sub * 16 + lh * 8;
      const int oa = buf * kOpHalves + (rb * 32 + l32) * kLS + ko;
      const int ob = buf * kOpHalves + (cb * 64 + l32) * kLS + ko;
      const h8 ahi = *(const h8*)(Ahi + oa);
      const h8 alo = *(const h8*)(Alo + oa);
      const h8 b0 = *(const h8*)(Bt + ob);
      const h8 b1 = *(const h8*)(Bt + ob + 32 * kLS);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, b1, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, b1, acc1, 0, 0, 0);
    }
    if (s + 1 < nsteps) stage(buf ^ 1);
    __syncthreads();
  }
  // RMSNorm row scales: the 4 threads of a staged row hold its partial sums
  if (g.gain) {
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if ((c.tid & 3) == 0) rs[srow] = 1.0f / __builtin_sqrtf(ss / (float)g.K + p.eps);
    __syncthreads();
  }
  // epilogue: accumulator register v of lane l holds tile row 32 rb + 8 (v / 4) + 4 (l / 32) + v % 4,
  // unit / column l % 32 of the wavefront's block
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
    const int pos = m0 + r;
    if (pos >= p.P) continue;
    float a = acc0[v], b = acc1[v];
    if (g.gain) {
      const float sc = rs[r];
      a *= sc;
      b *= sc;
    }
    if (g.ep == EPI_RESID) {
      const int n = tn * kTN + cb * 64 + l32;
      float* xo = g.out + (int64_t)pos * g.ld_out;
      if (n < g.n_out) *gp(xo + n) += a;
      if (n + 32 < g.n_out) *gp(xo + n + 32) += b;
    } else if (g.ep == EPI_UG) {
      const int u = tn * 64 + cb * 32 + l32;
      if (u < g.n_out) *gp(g.out + (int64_t)pos * g.ld_out + u) = a / (1.0f + __expf(-a)) * b;
    } else {
      const int u = tn * 64 + cb * 32 + l32;
      if (u >= g.n_out) continue;
      const int hh = p.hd >> 1, head = u / hh, i = u - head * hh;
      if (head < p.nq + p.nkv) {  // q or k head: rotate the pair (i, i + hd/2) by the position's angle
        const float* cs = p.rope + ((int64_t)pos * hh + i) * 2;
        const float co = *gp(cs), sn = *gp(cs + 1);
        const float ra = a * co - b * sn, rb2 = a * sn + b * co;
        a = ra;
        b = rb2;
      }
      if (head < p.nq) {
        float* qo = p.Q + (int64_t)pos * p.nq * p.hd + head * p.hd + i;
        *gp(qo) = a;
        *gp(qo + hh) = b;
      } else {
        const bool isk = head < p.nq + p.nkv;
        const int kvh = head - p.nq - (isk ? 0 : p.nkv);
        uint16_t* dst = (isk ? p.kc : p.vc) + (((int64_t)g.layer * p.nkv + kvh) * p.max_seq + pos) * p.hd + i;
        *gp(dst) = __builtin_bit_cast(uint16_t, (_Float16)a);
        *gp(dst + hh) = __builtin_bit_cast(uint16_t, (_Float16)b);
      }
    }
  }
  __syncthreads();  // the staging buffers and scales are reused by the next tile
}

// Work distribution of a stage whose items a whole workgroup processes.
// Static: workgroup c takes items c, c + grid, ...  Dynamic (a work queue,
// "8 - Ecrire son megakernel", section 8.8): the workgroup claims its next
// item from the stage's counter while it works on the current one, so a
// workgroup that finishes early takes more items.
template <typename F>
__device__ __forceinline__ void wg_items(PCx& c, int items, F&& work) {
  const PParams& p = *c.pp;
  if (!p.dynamic) {
    for (int t = c.cta; t < items; t += c.grid) work(t);
    return;
  }
  int* slot = (int*)(pf_smem + kClaimOff);
  uint32_t* ctr = p.queue + c.epoch;
  if (c.tid == 0) *slot = (int)__hip_atomic_fetch_add(gp(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  int t = *slot;
  __syncthreads();
  while (t < items) {
    uint32_t nxt = 0;
    if (c.tid == 0) nxt = __hip_atomic_fetch_add(gp(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    work(t);
    if (c.tid == 0) *slot = (int)nxt;
    __syncthreads();
    t = *slot;
    __syncthreads();
  }
}

__device__ __forceinline__ void gemm_stage(PCx& c, const Gemm& g) {
  const int n_tm = (c.pp->P + kTM - 1) / kTM;
  const int n_tn = g.ep == EPI_RESID ? (g.n_out + kTN - 1) / kTN : (g.n_out + 63) / 64;
  // consecutive items are the row tiles of one weight tile: workgroups working at the same time share its weight rows in L2
  wg_items(c, n_tm * n_tn, [&](int t) { gemm_tile(c, g, t % n_tm, t / n_tm); });
}

// ---------------------------------------------------------------- causal attention
// Work item: query head h and a block of 16 positions.  Wavefront w takes
// positions p0 + 4 (w % 4) .. + 4 (one per 16-lane row; lane i of a row holds
// dims [i * HD/16, (i+1) * HD/16)) and the key blocks of parity w / 4; each
// keeps an online softmax in the exp2 domain (q pre-scaled by log2(e)/sqrt(hd))
// and the two key halves are merged through LDS.  Query p attends keys 0..p.
template <int HD>
__device__ void att_stage(PCx& c, int l) {
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
      *gp(p.O + (int64_t)pos * p.nq * HD + h * HD + dd) = (a0 * r0[2 + dd] + a1 * r1[2 + dd]) / (a0 * r0[1] + a1 * r1[1]);
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
__device__ __attribute__((noinline)) void att_stage_mfma(PCx& c, int l) {
  constexpr int KS = HD / 16;  // MFMA K-steps over the head dims
  constexpr int DB = HD / 32;  // 32-dim blocks of O^T
  const PParams& p = *c.pp;
  const int P = p.P, nqb = (P + 31) / 32, items = p.nq * nqb;
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
    const int qb = nqb - 1 - it / p.nq, h = it - (it / p.nq) * p.nq;
    const int g = h * p.nkv / p.nq;
    const int q0 = qb * 32, pq = q0 + i32;           // this lane's query
    const int lim = min(pq, P - 1);                  // last key it attends
    const int kmax = min(q0 + 31, P - 1);            // last key of any query of the block
    // Q^T operands: dims 16 s + 8 hh + e of query pq, as hi and lo halves
    h8 qh[KS], ql[KS];
    {
      const float* qrow = p.Q + (int64_t)min(pq, P - 1) * p.nq * HD + h * HD + 8 * hh;
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
    const int64_t hbase = ((int64_t)l * p.nkv + g) * p.max_seq * HD;
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
      float* orow = p.O + (int64_t)pq * p.nq * HD + h * HD;
      const float inv = 1.0f / lt;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          // dims 32 b + 8 a + 4 hh + {0..3}: registers 4 a .. 4 a + 3
          const f4 v = {o[b][4 * a] * inv, o[b][4 * a + 1] * inv, o[b][4 * a + 2] * inv, o[b][4 * a + 3] * inv};
          *gp((f4*)(orow + 32 * b + 8 * a + 4 * hh)) = v;
        }
    }
    it = p.dynamic ? __builtin_amdgcn_readfirstlane(nxt_raw) : nxt_raw;
  }
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
  // the residual stream starts as the embedding rows of the prompt
  {
    const int64_t n = (int64_t)p.P * p.d;
    for (int64_t i = (int64_t)c.cta * kPT + c.tid; i < n; i += (int64_t)c.grid * kPT) {
      const int64_t pos = i / p.d, k = i - pos * p.d;
      *gp(p.X + i) = (float)__builtin_bit_cast(_Float16, *gp(p.embed + (int64_t)*gp(p.ids + pos) * p.d + k));
    }
  }
  if (grid_barrier(c, OP_QKV, 0)) return;
  const int qd = p.nq * p.hd, kvd = p.nkv * p.hd;
  const int64_t per_layer = (int64_t)(qd + 2 * kvd) * p.d + (int64_t)p.d * qd + 3LL * p.f * p.d;
  for (int l = 0; l < p.L; ++l) {
    const uint16_t* wl = p.canon + l * per_layer;
    const uint16_t* wo = wl + (int64_t)(qd + 2 * kvd) * p.d;
    const uint16_t* wg = wo + (int64_t)p.d * qd;
    const uint16_t* wu = wg + (int64_t)p.f * p.d;
    const uint16_t* wd = wu + (int64_t)p.f * p.d;
    const uint16_t* g1 = p.norms + (int64_t)l * 2 * p.d;
    const uint16_t* g2 = g1 + p.d;
    gemm_stage(c, Gemm{EPI_QKV, l, p.X, p.d, p.d, g1, wl, (p.nq + 2 * p.nkv) * (p.hd / 2), nullptr, 0, nullptr});
    if (grid_barrier(c, OP_QKV, l)) return;
    if (p.hd == 64) att_stage_mfma<64>(c, l);
    else if (p.hd == 128) att_stage_mfma<128>(c, l);
    else att_stage<256>(c, l);
    if (grid_barrier(c, OP_ATT, l)) return;
    gemm_stage(c, Gemm{EPI_RESID, l, p.O, qd, qd, nullptr, wo, p.d, p.X, p.d, nullptr});
    if (grid_barrier(c, OP_OPROJ, l)) return;
    gemm_stage(c, Gemm{EPI_UG, l, p.X, p.d, p.d, g2, wg, p.f, p.M, p.f, wu});
    if (grid_barrier(c, OP_UPGATE, l)) return;
    gemm_stage(c, Gemm{EPI_RESID, l, p.M, p.f, p.f, nullptr, wd, p.d, p.X, p.d, nullptr});
    if (grid_barrier(c, OP_DOWN, l)) return;
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
