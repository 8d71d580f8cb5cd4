// mk_layout.h -- data layouts shared by the host planner and the device
// interpreter: instruction records, kernel parameters, GEMV work split and
// the sentinel bit patterns.
#pragma once
#include <stdint.h>

#if defined(__HIP__)
#define MK_HD __host__ __device__ inline
#else
#define MK_HD inline
#endif

namespace mk {

#ifndef MK_WAVES
#define MK_WAVES 8
#endif
constexpr int kWaves = MK_WAVES;          // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;     // 512 threads
#ifndef MK_RING
#define MK_RING 12
#endif
constexpr int kRing = MK_RING;            // 1 KB weight chunks in flight per wavefront (LDS ring)
constexpr int kChunkHalfs = 512;          // fp16 values per chunk = 64 lanes x 8
constexpr int kMaxK = 16384;              // longest GEMV row
constexpr int kRedDims = 8;               // output dims per attention-reduce unit
constexpr int kScratchFloats = 4352;      // LDS scratch for cross-wave reductions (17 KB)
constexpr int kResidRows = 1024;          // LDS rows for residual inputs / staged GEMV outputs
constexpr int kMaxTopK = 16;              // largest k of top-k sampling
constexpr int kPosBatch = 4;              // positions per wavefront of a short attention split
constexpr int kShortSplitMax = kPosBatch * kWaves;  // longer splits take the long-split path

// Small LDS fields after the residual rows (byte offsets within a 1 KB block).
constexpr int kSmallBytes = 1024;
constexpr int kOffFlags = 0;              // u32 [2][kWaves] failure flags (double-buffered)
constexpr int kOffWsum = 64;              // f32 [kWaves] partial sums of squares
constexpr int kOffKeys = 96;              // u64 [kWaves] argmax keys
constexpr int kOffMisc = 160;             // u32 [16] trace scratch
static_assert(kOffMisc + 64 <= kSmallBytes, "small LDS fields overflow");

// Sentinels: bit patterns no computed value takes.  A quiet NaN whose low
// payload bits can come neither from arithmetic (default NaN 0x7FC00000) nor
// from widening an fp16 value (low 13 bits zero).
constexpr uint32_t kSent32 = 0x7FC05E17u;
constexpr uint16_t kSent16 = 0x7E17u;     // fp16 quiet NaN with a payload
constexpr uint64_t kSent64 = 0;           // argmax keys are never 0

enum Op : uint8_t {
  OP_END = 0,
  OP_QKV = 1,     // RMSNorm + fused QKV GEMV + RoPE, K/V into the cache
  OP_ATT = 2,     // split attention partials (m, l, o) per (kv head, split)
  OP_RED = 3,     // (unused: the last split of each kv head merges them inside OP_ATT)
  OP_OPROJ = 4,   // x += Wo o
  OP_UPGATE = 5,  // RMSNorm + gate/up GEMV + silu(g) * u
  OP_DOWN = 6,    // x += Wd m
  OP_LMHEAD = 7,  // final RMSNorm + LM head GEMV + per-workgroup argmax
  OP_ARGMAX = 8,  // every workgroup merges the per-workgroup argmax keys
  OP_CHAIN = 9,   // GEMV-tanh chain stage
};

// One instruction of a workgroup's list (32 bytes).
struct Ins {
  uint8_t op;
  uint8_t upr;       // rows per GEMV unit (2 for rotary / gate-up pairs)
  uint8_t ks;        // K slices across wavefronts
  uint8_t cps;       // 512-wide chunks per slice
  int16_t layer;
  int16_t sync_in;   // stage consumed (counter mode), -1 none
  int16_t sync_out;  // stage produced, -1 none
  int16_t n_in;      // producers of sync_in per step
  int32_t u0;        // first global unit
  int32_t nu;        // number of units
  int32_t slot;      // argmax slot of this workgroup (LM head)
  int32_t kpad;      // padded GEMV row length (columns staged in LDS)
  int32_t pad;
};
static_assert(sizeof(Ins) == 32, "Ins must be 32 bytes");

// The attention stage's part of the staged vector (floats): q [G][hd] and
// the current position's K and V rows, rounded up to 1 KB, then one 4 KB K/V
// ring per wavefront for long splits (two position groups of 1 KB of K and
// 1 KB of V, filled by DMA).
MK_HD int att_ring_offset(int G, int hd) { return ((G + 2) * hd + 255) / 256 * 256; }
MK_HD int att_stage_floats(int G, int hd) { return att_ring_offset(G, hd) + kWaves * 1024; }

// GEMV split inside one workgroup: units are dealt round-robin to kWaves/ks
// row groups; each row's chunks are split into ks slices of cps chunks.
MK_HD int units_of_group(int nu, int rg, int gi) { return nu > gi ? (nu - gi + rg - 1) / rg : 0; }

struct Buf {            // an activation buffer [epoch][layer][replica][n]
  float* p;
  int64_t es, ls, rs;   // element strides
};

struct Fault {
  int32_t code, cta, pc, op, step, layer, index, pad;
};

// Kernel parameters (passed by value).
struct KParams {
  // program
  const Ins* ins;
  const int32_t* ins_off;     // [grid + 1]
  int32_t n_steps, pos0, first_token, chain;
  const int32_t* forced;      // [n_steps] or null
  int32_t* tokens;            // [n_steps]
  float* logits;              // [n_steps][V] or null
  // weights
  const uint8_t* stream;      // repacked weight chunks
  const int64_t* wave_off;    // [grid * kWaves] chunk offsets
  const int32_t* wave_n;      // [grid * kWaves] chunks per step
  const uint16_t* embed;      // [V][d]
  const uint16_t* norms;      // [L][2][d] then final [d]
  const float* rope;          // [max_seq][hd/2][2] (cos, sin)
  uint16_t* kc;               // [L][nkv][max_seq][hd]
  uint16_t* vc;
  // activations and sync
  Buf xa, xm, q, o, m, y;
  float* att_o;               // [3][L][nq][S][hd]
  float* att_ml;              // [3][L][nq][S][2]
  uint32_t* att_cnt;          // [L][nkv] splits finished (zero at launch, monotonic)
  uint64_t* lmp;              // [3][R][lm_slots]
  int64_t lmp_es, lmp_rs;
  const float* x0;            // chain input
  uint32_t* counters;         // [n_sync_ids]
  Fault* fault;
  uint32_t* abort_flag;
  uint32_t* trace;            // [grid][trace_steps][max_ins][8]
  uint32_t* progress;         // [grid]: (step << 16) | (pc + 1) of the last finished instruction
  uint64_t* ts;               // [grid][max_ins][8] fine timestamps of step 0 (diagnostics), or null
  int32_t trace_steps, max_ins;
  // dims
  int32_t L, d, nq, nkv, hd, f, V, max_seq, S, R, sync_mode, lm_slots;
  int32_t chain_n, vec_floats;
  float eps;
  uint64_t watchdog_ticks;    // 100 MHz ticks
  int32_t poll_sleep;         // s_sleep units between failed poll rounds (0 = spin)
  int32_t stall_cta;          // diagnostics: this workgroup waits on stall_word in step 0 (-1: none)
  // top-k / temperature sampling (top_k == 1: greedy argmax, the lists are unused)
  uint64_t* lmk;              // [3][R][lm_slots][kMaxTopK] per-workgroup top-k keys
  int64_t lmk_es, lmk_rs;
  int32_t top_k;
  float inv_temp;             // 1 / temperature
  uint32_t seed_lo, seed_hi;  // Philox key
  const uint32_t* stall_word; // a sync word the host leaves at the sentinel (see stall_cta)
};

// ---------------------------------------------------------------- prompt prefill
// Parameters of the prefill kernel (mk_prefill.hip): positions [0, P) of a
// prompt through every layer with MFMA GEMMs, filling the KV cache.
struct PParams {
  int32_t L, d, nq, nkv, hd, f, max_seq, P;
  float eps;
  int32_t pad0;
  const uint16_t* canon;    // per layer [wq; wk; wv] [(nq + 2 nkv) hd][d], wo [d][nq hd], wg, wu [f][d], wd [d][f]
  const uint16_t* norms;    // [L][2][d]
  const uint16_t* embed;    // [V][d]
  const int32_t* ids;       // [P]
  const float* rope;        // [max_seq][hd/2][2] (cos, sin)
  uint16_t* kc;             // [L][nkv][max_seq][hd]
  uint16_t* vc;
  float* X;                 // [P][d] residual stream
  float* Q;                 // [P][nq hd] rotated queries
  // GEMM A operands as fp16 hi + lo halves of fp32 values (a = hi + lo to 2^-22), written by their
  // producers; rows padded with zeros to a multiple of 32 columns
  uint16_t* Oh;             // [P][ldo] attention output, hi halves
  uint16_t* Ol;             //          lo halves
  uint16_t* Mh;             // [P][ldm] silu(gate) * up
  uint16_t* Ml;
  uint16_t* Xh;             // [P][d] x times the gain of the next RMSNorm
  uint16_t* Xl;
  float* ssp;               // [ceil(d / 64)][P] sums of x^2 over 64-column blocks (for 1 / rms)
  int32_t ldo, ldm;
  uint32_t* barrier;        // grid barrier counter (zero at launch)
  uint32_t* abort_flag;
  Fault* fault;
  uint32_t* progress;       // [grid]: stages finished by each workgroup
  uint64_t watchdog_ticks;  // 100 MHz ticks per wait
  uint64_t* marks;          // [1 + 5 L]: device clock when workgroup 0 left each grid barrier, or null
  uint32_t* queue;          // [1 + 5 L] work-queue counters, one per stage (zero at launch)
  int32_t dynamic;          // 1: workgroups / wavefronts claim their tiles from the queue; 0: static deal
  int32_t pad1;
  float* part;              // split-K partial tiles [grid][kPartFloats]; in the attention stage of short
                            // prompts the key chunks' partials [2 grid][kAttPartFloats]
  uint32_t* tile_cnt;       // [grid] split-K arrivals per output tile (zero at launch and between stages)
};
// One split-K partial: a tile of up to 128 x 256 fp32 accumulators.
constexpr int kPartFloats = 128 * 256;
// one attention key chunk's partial: 8 wavefronts x 64 lanes x (m, l and head_dim 128's 4 x 16 O^T values)
constexpr int kAttPartFloats = 8 * 64 * (2 + 4 * 16);

}  // namespace mk
