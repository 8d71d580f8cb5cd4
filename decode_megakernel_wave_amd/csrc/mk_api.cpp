// mk_api.cpp -- the C ABI: context lifecycle, weight repacking, launches.
//
// The launcher follows the one-wave rule of "8 - Ecrire son megakernel"
// (section 8.3): set the dynamic LDS size, query how many workgroups fit on a
// CU, launch exactly CUs x occupancy workgroups and refuse to launch when the
// kernel does not fit (launching more would deadlock silently).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_diag.h"
#include "mk_layout.h"
#include "mk_plan.h"

using namespace mk;

extern "C" {
hipError_t mk_launch_monokernel(const KParams* kp_dev, int grid, int lds_bytes, hipStream_t s);
hipError_t mk_kernel_attributes(int lds_bytes, int* occupancy);
hipError_t mk_launch_monokernel_w4h128(const KParams* kp_dev, int grid, int lds_bytes, hipStream_t s);
hipError_t mk_kernel_attributes_w4h128(int lds_bytes, int* occupancy);
hipError_t mk_launch_monokernel_w4h128_ctr(const KParams* kp_dev, int grid, int lds_bytes, hipStream_t s);
hipError_t mk_kernel_attributes_w4h128_ctr(int lds_bytes, int* occupancy);
hipError_t mk_launch_monokernel_w4h128_long(const KParams* kp_dev, int grid, int lds_bytes, hipStream_t s);
hipError_t mk_kernel_attributes_w4h128_long(int lds_bytes, int* occupancy);
hipError_t mk_launch_fill32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
hipError_t mk_launch_fill_kv(uint16_t* kc, uint16_t* vc, int64_t rows, int max_seq, int hd, int p0, int p1, hipStream_t s);
hipError_t mk_launch_gather(uint16_t* dst, const void* desc, int64_t n_chunks, hipStream_t s);
hipError_t mk_launch_count32(const uint32_t* p, int64_t n, uint32_t v, unsigned long long* out, hipStream_t s);
hipError_t mk_launch_count_kv(const uint16_t* kc, const uint16_t* vc, int64_t rows, int max_seq, int hd, int p0, int p1,
                              unsigned long long* out, hipStream_t s);
hipError_t mk_launch_probe_empty(hipStream_t s);
hipError_t mk_launch_probe_read(const void* p, int64_t n16, void* sink, int grid, hipStream_t s);
hipError_t mk_launch_probe_barrier(uint32_t* counter, int rounds, uint64_t deadline_ticks, uint64_t* out, int grid,
                                   hipStream_t s);
hipError_t mk_probe_barrier_occupancy(int* occupancy);
hipError_t mk_launch_probe_handoff(const void* buf, uint32_t n_chunks, int mode, int same_xcd, int rounds,
                                   int stream_chunks, uint32_t* flags, uint64_t* ticks, int32_t* xcc,
                                   uint32_t* timeouts, void* sink, int grid, hipStream_t s);
hipError_t mk_probe_handoff_occupancy(int* occupancy);
int mk_probe_handoff_pairs();
hipError_t mk_launch_count64(const uint64_t* p, int64_t n, int stride, int width, uint64_t v, unsigned long long* out,
                             hipStream_t s);
hipError_t mk_scratch_address(int device, void** out, size_t* bytes);
int mk_prefill_lds_bytes(int hd);
hipError_t mk_prefill_attributes(int lds_bytes, int* occupancy);
hipError_t mk_launch_prefill(const PParams* pp_dev, int grid, int lds_bytes, hipStream_t s);
}

namespace {

thread_local std::string g_create_error;

struct GatherDesc {
  const uint16_t* src;
  int32_t valid;
  int32_t pad;
};

enum State { ST_CREATED = 0, ST_LOADED = 1, ST_READY = 2 };

// Device memory shared by the decoder and the chain.
struct Engine {
  int device = 0;
  hipStream_t stream = nullptr;
  mk_options opt{};
  Plan plan;
  int n_cu = 0, occ = 0, grid = 0;
  bool spec = false;  // every instruction fits the kernel specialised to 4-chunk slices and head_dim 128
  int last_kind = -1;  // the kernel the last launch ran (kernel_kind), -1 before any
  std::string err;
  // device buffers
  uint8_t* d_stream = nullptr;
  Ins* d_ins = nullptr;
  int32_t* d_ins_off = nullptr;
  int64_t* d_wave_off = nullptr;
  int32_t* d_wave_n = nullptr;
  float* d_arena = nullptr;
  int64_t arena_words = 0, lmp_word_off = 0;
  uint32_t* d_counters = nullptr;
  Fault* d_fault = nullptr;
  uint32_t* d_abort = nullptr;
  uint32_t* d_trace = nullptr;
  uint32_t* d_progress = nullptr;
  uint64_t* d_ts = nullptr;
  uint32_t* d_stall = nullptr;  // a word left at the sentinel for the failure-path test
  int stall_cta = -1;           // armed for the next launch only
  int64_t trace_words = 0;
  int32_t* d_tokens = nullptr;
  int32_t* d_forced = nullptr;
  float* d_logits = nullptr;
  int64_t logits_cap = 0;
  KParams* d_kp = nullptr;
  KParams h_kp{};
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  mk_stats_t last{};
  std::vector<void*> allocs;

  int fail(int code, const std::string& msg) {
    err = msg;
    return code;
  }
  int hip_fail(hipError_t e, const char* what) {
    err = std::string(what) + ": " + hipGetErrorString(e);
    return MK_EHIP;
  }
  template <typename T>
  int alloc(T** p, size_t bytes) {
    void* q = nullptr;
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(&q, bytes);
    if (e != hipSuccess) {
      err = "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e);
      return MK_ENOMEM;
    }
    allocs.push_back(q);
    *p = (T*)q;
    return MK_OK;
  }
  void release() {
    if (stream) hipStreamSynchronize(stream);
    for (void* p : allocs) hipFree(p);
    allocs.clear();
    if (ev0) hipEventDestroy(ev0);
    if (ev1) hipEventDestroy(ev1);
    ev0 = ev1 = nullptr;
  }
};

#define HIPCHK(eng, x)                                       \
  do {                                                       \
    hipError_t e_ = (x);                                     \
    if (e_ != hipSuccess) return (eng).hip_fail(e_, #x);     \
  } while (0)
#define CHK(x)                 \
  do {                         \
    int r_ = (x);              \
    if (r_ != MK_OK) return r_; \
  } while (0)

int sanitize_options(const mk_options* in, mk_options* out) {
  mk_default_options(out);
  if (in) *out = *in;
  if (out->sync_mode != MK_SYNC_SENTINEL && out->sync_mode != MK_SYNC_COUNTER) return MK_EINVAL;
  if (!(out->xcd_replicas == 1 || out->xcd_replicas == 2 || out->xcd_replicas == 4 || out->xcd_replicas == 8)) return MK_EINVAL;
  if (out->attn_splits < 0 || out->attn_splits > 64) return MK_EINVAL;
  if (out->trace_steps < 0 || out->watchdog_us <= 0 || out->grid < 0) return MK_EINVAL;
  if (out->work_queue != 0 && out->work_queue != 1) return MK_EINVAL;
  return MK_OK;
}

// Device, occupancy and grid (the one-wave launch).
int engine_setup(Engine& g, int device, void* stream, const mk_options* opts, int lds_bytes) {
  if (sanitize_options(opts, &g.opt) != MK_OK) return g.fail(MK_EINVAL, "invalid options");
  g.device = device;
  g.stream = (hipStream_t)stream;
  int ndev = 0;
  HIPCHK(g, hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev) return g.fail(MK_EINVAL, "no such device");
  HIPCHK(g, hipSetDevice(device));
  hipDeviceProp_t prop;
  HIPCHK(g, hipGetDeviceProperties(&prop, device));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return g.fail(MK_EINVAL, std::string("the kernels are built for gfx950, device is ") + prop.gcnArchName);
  g.n_cu = prop.multiProcessorCount;
  if (lds_bytes > (int)prop.sharedMemPerBlock) return g.fail(MK_EOCC, "LDS footprint exceeds the per-workgroup limit");
  HIPCHK(g, mk_kernel_attributes(lds_bytes, &g.occ));
  int occ_spec = 0, occ_ctr = 0, occ_long = 0;
  HIPCHK(g, mk_kernel_attributes_w4h128(lds_bytes, &occ_spec));
  HIPCHK(g, mk_kernel_attributes_w4h128_ctr(lds_bytes, &occ_ctr));
  HIPCHK(g, mk_kernel_attributes_w4h128_long(lds_bytes, &occ_long));
  g.occ = std::min({g.occ, occ_spec, occ_ctr, occ_long});  // any of the kernels may run this grid
  if (g.occ < 1) return g.fail(MK_EOCC, "the monokernel does not fit on a CU (occupancy 0)");
  const int wave = g.n_cu * g.occ;
  g.grid = g.opt.grid > 0 ? g.opt.grid : wave;
  if (g.grid > wave) return g.fail(MK_EOCC, "requested grid exceeds CUs x occupancy: workgroups would not all be resident");
  HIPCHK(g, hipEventCreate(&g.ev0));
  HIPCHK(g, hipEventCreate(&g.ev1));
  return MK_OK;
}

// True when the kernel specialised to 4-chunk GEMV slices, head_dim 128 and two
// query heads per kv head runs
// every instruction of the plan exactly as the general one does.
bool fits_specialised(const Plan& p) {
  if (!p.dm.chain && (p.dm.hd != 128 || p.dm.nq != 2 * p.dm.nkv)) return false;
  for (const Ins& in : p.ins) {
    const bool gemv = in.op == OP_QKV || in.op == OP_OPROJ || in.op == OP_UPGATE || in.op == OP_DOWN ||
                      in.op == OP_LMHEAD || in.op == OP_CHAIN;
    if (gemv && in.cps != 4) return false;
  }
  return true;
}

int upload_plan(Engine& g) {
  const Plan& p = g.plan;
  g.spec = fits_specialised(p);
  CHK(g.alloc(&g.d_ins, p.ins.size() * sizeof(Ins)));
  CHK(g.alloc(&g.d_ins_off, p.ins_off.size() * sizeof(int32_t)));
  CHK(g.alloc(&g.d_wave_off, p.wave_off.size() * sizeof(int64_t)));
  CHK(g.alloc(&g.d_wave_n, p.wave_n.size() * sizeof(int32_t)));
  CHK(g.alloc(&g.d_stream, (size_t)p.stream_bytes()));
  HIPCHK(g, hipMemcpy(g.d_ins, p.ins.data(), p.ins.size() * sizeof(Ins), hipMemcpyHostToDevice));
  HIPCHK(g, hipMemcpy(g.d_ins_off, p.ins_off.data(), p.ins_off.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  HIPCHK(g, hipMemcpy(g.d_wave_off, p.wave_off.data(), p.wave_off.size() * sizeof(int64_t), hipMemcpyHostToDevice));
  HIPCHK(g, hipMemcpy(g.d_wave_n, p.wave_n.data(), p.wave_n.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  CHK(g.alloc(&g.d_counters, std::max(1, p.n_sync) * sizeof(uint32_t)));
  CHK(g.alloc(&g.d_fault, sizeof(Fault)));
  CHK(g.alloc(&g.d_abort, sizeof(uint32_t)));
  CHK(g.alloc(&g.d_stall, sizeof(uint32_t)));
  CHK(g.alloc(&g.d_kp, sizeof(KParams)));
  CHK(g.alloc(&g.d_progress, (size_t)g.grid * 4));
  CHK(g.alloc(&g.d_ts, (size_t)g.grid * p.max_ins * 8 * 8));
  if (g.opt.trace_steps > 0) {
    g.trace_words = (int64_t)g.grid * g.opt.trace_steps * p.max_ins * 8;
    CHK(g.alloc(&g.d_trace, g.trace_words * 4));
  }
  return MK_OK;
}

// Repack weights: every chunk of every wavefront stream from its source row.
int repack(Engine& g, const std::vector<const uint16_t*>& mats) {
  const Plan& p = g.plan;
  const int64_t n = (int64_t)p.chunks.size();
  if (n == 0) return MK_OK;
  std::vector<GatherDesc> desc(n);
  for (int64_t i = 0; i < n; ++i) {
    const ChunkSrc& s = p.chunks[i];
    const int cols = p.mat_cols(s.mat);
    const uint16_t* base = mats[s.mat];
    if (!base) return g.fail(MK_EINVAL, "a weight pointer is NULL");
    desc[i].src = base + (int64_t)s.row * cols + (int64_t)s.cc * kChunkHalfs;
    desc[i].valid = std::max(0, std::min(kChunkHalfs, cols - s.cc * kChunkHalfs));
    desc[i].pad = 0;
  }
  void* d_desc = nullptr;
  hipError_t e = hipMalloc(&d_desc, desc.size() * sizeof(GatherDesc));
  if (e != hipSuccess) return g.fail(MK_ENOMEM, "hipMalloc for the repack table failed");
  e = hipMemcpyAsync(d_desc, desc.data(), desc.size() * sizeof(GatherDesc), hipMemcpyHostToDevice, g.stream);
  if (e == hipSuccess) e = mk_launch_gather((uint16_t*)g.d_stream, d_desc, n, g.stream);
  if (e == hipSuccess) e = hipStreamSynchronize(g.stream);
  hipFree(d_desc);
  if (e != hipSuccess) return g.hip_fail(e, "weight repack");
  return MK_OK;
}

void fill_common_params(Engine& g, KParams& k) {
  const Plan& p = g.plan;
  k.ins = g.d_ins;
  k.ins_off = g.d_ins_off;
  k.stream = g.d_stream;
  k.wave_off = g.d_wave_off;
  k.wave_n = g.d_wave_n;
  k.counters = g.d_counters;
  k.fault = g.d_fault;
  k.abort_flag = g.d_abort;
  k.trace = g.d_trace;
  k.progress = g.d_progress;
  k.ts = getenv("MK_DEBUG_TS") ? g.d_ts : nullptr;
  k.trace_steps = g.opt.trace_steps;
  k.max_ins = p.max_ins;
  k.S = p.S;
  k.R = p.R;
  k.sync_mode = p.sync_mode;
  k.lm_slots = p.lm_slots;
  k.watchdog_ticks = (uint64_t)g.opt.watchdog_us * 100ull;  // 100 MHz wall clock
  k.poll_sleep = getenv("MK_POLL_SLEEP") ? atoi(getenv("MK_POLL_SLEEP")) : 0;
  k.stall_cta = g.stall_cta;
  k.stall_word = g.d_stall;
}

// Which monokernel a launch whose first step decodes position pos0 runs: 0
// general, 1 specialised (sentinel sync), 2 specialised (counter sync), 3
// specialised with the DMA-fed long attention splits, taken when every split
// of the first step is already longer than the short path's bound (the
// context only grows within a launch; a short last split still takes the
// short path there).  MK_GENERAL_KERNEL=1 forces the general kernel
// (comparison runs).
int kernel_kind(const Engine& g, int pos0) {
  if (!g.spec || getenv("MK_GENERAL_KERNEL")) return 0;
  if (g.plan.sync_mode != 0) return 2;
  const int64_t T = (int64_t)pos0 + 1;
  const bool long_splits = !g.plan.dm.chain && (T + g.plan.S - 1) / g.plan.S > kShortSplitMax;
  return long_splits ? 3 : 1;
}

// Reset sync state, launch once, wait, collect the fault record.
int launch(Engine& g, KParams& k, int n_steps) {
  HIPCHK(g, mk_launch_fill32(g.d_counters, std::max(1, g.plan.n_sync), 0u, g.stream));
  HIPCHK(g, mk_launch_fill32((uint32_t*)g.d_fault, sizeof(Fault) / 4, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32(g.d_abort, 1, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32(g.d_progress, g.grid, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32(g.d_stall, 1, kSent32, g.stream));
  g.stall_cta = -1;  // one launch only
  if (g.d_trace) HIPCHK(g, mk_launch_fill32(g.d_trace, g.trace_words, 0u, g.stream));
  g.h_kp = k;
  HIPCHK(g, hipMemcpyAsync(g.d_kp, &g.h_kp, sizeof(KParams), hipMemcpyHostToDevice, g.stream));
  HIPCHK(g, hipEventRecord(g.ev0, g.stream));
  const int kind = kernel_kind(g, k.chain ? 0 : k.pos0);
  g.last_kind = kind;
  if (kind == 0) HIPCHK(g, mk_launch_monokernel(g.d_kp, g.grid, g.plan.lds_bytes, g.stream));
  else if (kind == 1) HIPCHK(g, mk_launch_monokernel_w4h128(g.d_kp, g.grid, g.plan.lds_bytes, g.stream));
  else if (kind == 2) HIPCHK(g, mk_launch_monokernel_w4h128_ctr(g.d_kp, g.grid, g.plan.lds_bytes, g.stream));
  else HIPCHK(g, mk_launch_monokernel_w4h128_long(g.d_kp, g.grid, g.plan.lds_bytes, g.stream));
  HIPCHK(g, hipEventRecord(g.ev1, g.stream));
  HIPCHK(g, hipStreamSynchronize(g.stream));
  float ms = 0.f;
  HIPCHK(g, hipEventElapsedTime(&ms, g.ev0, g.ev1));
  Fault f{};
  HIPCHK(g, hipMemcpy(&f, g.d_fault, sizeof(Fault), hipMemcpyDeviceToHost));
  g.last.gpu_ms = ms;
  g.last.steps = n_steps;
  g.last.grid = g.grid;
  g.last.block = kThreads;
  g.last.lds_bytes = g.plan.lds_bytes;
  g.last.ring_depth = kRing;
  g.last.stream_bytes = g.plan.stream_bytes();
  g.last.weight_bytes = g.plan.weight_bytes;
  g.last.n_cu = g.n_cu;
  g.last.occupancy = g.occ;
  memcpy(&g.last.fault, &f, sizeof(Fault));
  if (f.code == MK_ETIMEOUT) {
    char buf[256];
    snprintf(buf, sizeof buf,
             "device watchdog: workgroup %d, instruction %d (op %d, layer %d, index %d), step %d waited too long",
             f.cta, f.pc, f.op, f.layer, f.index, f.step);
    std::string msg = buf;
    // where every workgroup stood: the slowest ones first
    std::vector<uint32_t> prog(g.grid);
    if (hipMemcpy(prog.data(), g.d_progress, prog.size() * 4, hipMemcpyDeviceToHost) == hipSuccess) {
      uint32_t lo = UINT32_MAX;
      for (uint32_t v : prog) lo = std::min(lo, v);
      int shown = 0;
      msg += "; least progress (step<<16|pc+1) " + std::to_string(lo) + " at workgroups";
      for (int i = 0; i < g.grid && shown < 16; ++i)
        if (prog[i] == lo) {
          msg += " " + std::to_string(i);
          ++shown;
        }
    }
    return g.fail(MK_ETIMEOUT, msg);
  }
  if (f.code == MK_ENAN) return g.fail(MK_ENAN, "a NaN logit was produced");
  return MK_OK;
}

}  // namespace

// ============================================================ decoder context
struct mk_ctx {
  Engine g;
  mk_config cfg{};
  int state = ST_CREATED;
  int pos = 0, next_tok = 0;
  std::vector<int32_t> hist;  // token consumed at each position
  int last_pos0 = 0, last_n = 0;
  // model buffers
  uint16_t* d_embed = nullptr;
  uint16_t* d_norms = nullptr;
  float* d_rope = nullptr;
  uint16_t* d_kc = nullptr;
  uint16_t* d_vc = nullptr;
  Buf xa{}, xm{}, q{}, o{}, m{};
  float* att_o = nullptr;
  float* att_ml = nullptr;
  uint32_t* att_cnt = nullptr;
  uint64_t* lmp = nullptr;
  int64_t lmp_es = 0, lmp_rs = 0;
  uint64_t* lmk = nullptr;
  int64_t lmk_es = 0, lmk_rs = 0;
  int top_k = 1, last_top_k = 1;
  float temperature = 1.0f;
  uint64_t seed = 0;
  int64_t layout[16] = {0};
  struct Region { int64_t off, words; };
  std::vector<Region> epoch_regions[3];  // per epoch: word ranges that a step fully writes
  // prompt prefill on MFMA (mk_prefill.hip)
  bool pf_ok = false;               // the shapes fit the prefill kernel
  int pf_grid = 0, pf_lds = 0;
  uint16_t* d_canon = nullptr;      // canonical weights, per layer [wq; wk; wv], wo, wg, wu, wd
  float *d_pX = nullptr, *d_pQ = nullptr, *d_pO = nullptr, *d_pM = nullptr;
  int32_t* d_pids = nullptr;
  uint32_t* d_pbar = nullptr;
  uint64_t* d_pmarks = nullptr;     // [1 + 5 L + 1]: start, then each grid barrier (device clock)
  uint32_t* d_pqueue = nullptr;     // [1 + 5 L] work-queue counters
  float* d_ppart = nullptr;         // split-K partial tiles, attention key-chunk partials
  float* d_pXhl = nullptr;          // [2][P][d] fp16 hi / lo halves of x times the next gain
  float* d_pssp = nullptr;          // [ceil(d / 64)][P] partial sums of squares of x
  int pf_ldo = 0, pf_ldm = 0;       // row strides (halves) of the attention-output and MLP planes
  uint32_t* d_ptile = nullptr;      // [grid] split-K arrival counters
  PParams* d_pp = nullptr;
  PParams h_pp{};
};

namespace {

int ctx_alloc_arena(mk_ctx* c) {
  Engine& g = c->g;
  const Plan& p = g.plan;
  const mk_config& k = c->cfg;
  const int L = k.n_layers, R = p.R, qd = k.n_heads * k.head_dim, S = p.S;
  int64_t off = 0;
  auto take = [&](Buf& b, int n, int reps) {
    b.rs = reps > 1 ? n : 0;
    b.ls = (int64_t)n * reps;
    b.es = b.ls * L;
    const int64_t o = off;
    for (int e = 0; e < 3; ++e) c->epoch_regions[e].push_back({o + e * b.es, b.es});
    off += ((3 * b.es + 63) / 64) * 64;
    return o;
  };
  const int64_t oxa = take(c->xa, k.d_model, R);
  const int64_t oxm = take(c->xm, k.d_model, R);
  const int64_t oq = take(c->q, qd, 1);
  const int64_t oo = take(c->o, qd, R);
  const int64_t om = take(c->m, k.ffn, R);
  const int64_t att_es = (int64_t)L * k.n_heads * S * k.head_dim;
  const int64_t oao = off;
  for (int e = 0; e < 3; ++e) c->epoch_regions[e].push_back({oao + e * att_es, att_es});
  off += ((3 * att_es + 63) / 64) * 64;
  const int64_t ml_es = (int64_t)L * k.n_heads * S * 2;
  const int64_t oml = off;
  for (int e = 0; e < 3; ++e) c->epoch_regions[e].push_back({oml + e * ml_es, ml_es});
  off += ((3 * ml_es + 63) / 64) * 64;
  g.lmp_word_off = off;
  c->lmp_rs = p.lm_slots;
  c->lmp_es = (int64_t)p.lm_slots * R;
  off += ((3 * c->lmp_es * 2 + 63) / 64) * 64;
  const int64_t ocnt = off;  // attention merge counters [L][n_kv_heads], zero at launch
  off += (((int64_t)L * k.n_kv_heads + 63) / 64) * 64;
  const int64_t olmk = off;  // per-workgroup top-k keys for sampling (u64, zero = not yet written)
  c->lmk_rs = (int64_t)p.lm_slots * kMaxTopK;
  c->lmk_es = c->lmk_rs * R;
  off += ((3 * c->lmk_es * 2 + 63) / 64) * 64;
  g.arena_words = off;
  const int64_t lay[11] = {oxa, oxm, oq, oo, om, oao, oml, g.lmp_word_off, off, ocnt, olmk};
  for (int i = 0; i < 11; ++i) c->layout[i] = lay[i];
  CHK(g.alloc(&g.d_arena, off * 4));
  float* a = g.d_arena;
  c->xa.p = a + oxa;
  c->xm.p = a + oxm;
  c->q.p = a + oq;
  c->o.p = a + oo;
  c->m.p = a + om;
  c->att_o = a + oao;
  c->att_ml = a + oml;
  c->lmp = (uint64_t*)(a + g.lmp_word_off);
  c->att_cnt = (uint32_t*)(a + ocnt);
  c->lmk = (uint64_t*)(a + olmk);
  return MK_OK;
}

// Buffers of the MFMA prefill, sized for a prompt of max_seq - 1 positions
// (the prompt's last token runs through the decode monokernel).  The prefill
// kernel needs every K dimension (d_model, n_heads * head_dim, ffn) to be a
// multiple of 8; other shapes prefill through the decode monokernel.
int ctx_alloc_prefill(mk_ctx* c) {
  Engine& g = c->g;
  const mk_config& k = c->cfg;
  const int qd = k.n_heads * k.head_dim, kvd = k.n_kv_heads * k.head_dim;
  // d_model a multiple of 32 and at most 8192: the normed GEMMs (K = d_model) take whole
  // 32-column steps and stage their gain in LDS; the GEMM tiles address an activation matrix
  // with 32-bit byte offsets
  const int64_t widest = std::max<int64_t>(std::max(k.d_model, k.ffn), qd);
  c->pf_ok = k.d_model % 32 == 0 && k.d_model <= 8192 && k.ffn % 8 == 0 && qd % 8 == 0 &&
             (int64_t)std::max(1, k.max_seq - 1) * widest * 4 < (1LL << 32);
  if (!c->pf_ok) return MK_OK;
  c->pf_lds = mk_prefill_lds_bytes(k.head_dim);
  int occ = 0;
  hipError_t e = mk_prefill_attributes(c->pf_lds, &occ);
  if (e != hipSuccess) return g.hip_fail(e, "prefill kernel attributes");
  if (occ < 1) {
    c->pf_ok = false;
    return MK_OK;
  }
  c->pf_grid = g.n_cu;  // one workgroup per CU: all resident, so the grid barriers cannot deadlock
  const int64_t P = std::max(1, k.max_seq - 1);
  const int64_t per_layer = (int64_t)(qd + 2 * kvd) * k.d_model + (int64_t)k.d_model * qd + 3LL * k.ffn * k.d_model;
  CHK(g.alloc(&c->d_canon, (size_t)per_layer * k.n_layers * 2));
  CHK(g.alloc(&c->d_pX, (size_t)P * k.d_model * 4));
  CHK(g.alloc(&c->d_pQ, (size_t)P * qd * 4));
  c->pf_ldo = (qd + 31) / 32 * 32;
  c->pf_ldm = (k.ffn + 31) / 32 * 32;
  CHK(g.alloc(&c->d_pO, (size_t)P * c->pf_ldo * 4));   // hi and lo planes
  CHK(g.alloc(&c->d_pM, (size_t)P * c->pf_ldm * 4));
  CHK(g.alloc(&c->d_pXhl, (size_t)P * k.d_model * 4));
  CHK(g.alloc(&c->d_pssp, (size_t)((k.d_model + 63) / 64) * P * 4));
  // the pad columns of the A planes stay zero (no producer writes them)
  HIPCHK(g, mk_launch_fill32((uint32_t*)c->d_pO, P * c->pf_ldo, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32((uint32_t*)c->d_pM, P * c->pf_ldm, 0u, g.stream));
  CHK(g.alloc(&c->d_pids, (size_t)P * 4));
  CHK(g.alloc(&c->d_pbar, 256));
  CHK(g.alloc(&c->d_pmarks, (size_t)(5 * k.n_layers + 2) * 8));
  CHK(g.alloc(&c->d_pqueue, (size_t)(5 * k.n_layers + 2) * 4));
  CHK(g.alloc(&c->d_ppart, (size_t)c->pf_grid * std::max(kPartFloats, 2 * kAttPartFloats) * 4));
  CHK(g.alloc(&c->d_ptile, (size_t)c->pf_grid * 4));
  CHK(g.alloc(&c->d_pp, sizeof(PParams)));
  return MK_OK;
}

// Positions [0, n) of a prompt through every layer in one launch of the
// prefill kernel (MFMA GEMMs, causal attention); fills the KV cache.
int ctx_prefill_mfma(mk_ctx* c, const int32_t* ids, int n) {
  Engine& g = c->g;
  const mk_config& k = c->cfg;
  HIPCHK(g, hipSetDevice(g.device));
  HIPCHK(g, hipMemcpyAsync(c->d_pids, ids, (size_t)n * 4, hipMemcpyHostToDevice, g.stream));
  HIPCHK(g, mk_launch_fill32(c->d_pbar, 1, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32((uint32_t*)g.d_fault, sizeof(Fault) / 4, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32(g.d_abort, 1, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32(g.d_progress, g.grid, 0u, g.stream));
  PParams& pp = c->h_pp;
  pp = PParams{};
  pp.L = k.n_layers;
  pp.d = k.d_model;
  pp.nq = k.n_heads;
  pp.nkv = k.n_kv_heads;
  pp.hd = k.head_dim;
  pp.f = k.ffn;
  pp.max_seq = k.max_seq;
  pp.P = n;
  pp.eps = k.rms_eps;
  pp.canon = c->d_canon;
  pp.norms = c->d_norms;
  pp.embed = c->d_embed;
  pp.ids = c->d_pids;
  pp.rope = c->d_rope;
  pp.kc = c->d_kc;
  pp.vc = c->d_vc;
  pp.X = c->d_pX;
  pp.Q = c->d_pQ;
  const int64_t Pa = std::max(1, k.max_seq - 1);
  pp.Oh = (uint16_t*)c->d_pO;
  pp.Ol = pp.Oh + Pa * c->pf_ldo;
  pp.Mh = (uint16_t*)c->d_pM;
  pp.Ml = pp.Mh + Pa * c->pf_ldm;
  pp.Xh = (uint16_t*)c->d_pXhl;
  pp.Xl = pp.Xh + Pa * k.d_model;
  pp.ssp = c->d_pssp;
  pp.ldo = c->pf_ldo;
  pp.ldm = c->pf_ldm;
  pp.barrier = c->d_pbar;
  pp.abort_flag = g.d_abort;
  pp.fault = g.d_fault;
  pp.progress = g.d_progress;
  pp.watchdog_ticks = (uint64_t)g.opt.watchdog_us * 100ull;
  pp.marks = c->d_pmarks;
  pp.queue = c->d_pqueue;
  pp.dynamic = g.opt.work_queue;
  pp.part = c->d_ppart;
  pp.tile_cnt = c->d_ptile;
  HIPCHK(g, mk_launch_fill32(c->d_pqueue, 5 * k.n_layers + 2, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32(c->d_ptile, c->pf_grid, 0u, g.stream));
  HIPCHK(g, mk_launch_fill32((uint32_t*)c->d_pmarks, 2 * (5 * k.n_layers + 2), 0u, g.stream));
  HIPCHK(g, hipMemcpyAsync(c->d_pp, &pp, sizeof(PParams), hipMemcpyHostToDevice, g.stream));
  HIPCHK(g, hipEventRecord(g.ev0, g.stream));
  HIPCHK(g, mk_launch_prefill(c->d_pp, c->pf_grid, c->pf_lds, g.stream));
  HIPCHK(g, hipEventRecord(g.ev1, g.stream));
  HIPCHK(g, hipStreamSynchronize(g.stream));
  float ms = 0.f;
  HIPCHK(g, hipEventElapsedTime(&ms, g.ev0, g.ev1));
  g.last.prefill_ms = ms;
  g.last.prefill_positions = n;
  g.last.prefill_grid = c->pf_grid;
  Fault f{};
  HIPCHK(g, hipMemcpy(&f, g.d_fault, sizeof(Fault), hipMemcpyDeviceToHost));
  memcpy(&g.last.fault, &f, sizeof(Fault));
  if (f.code == MK_ETIMEOUT) {
    char buf[160];
    snprintf(buf, sizeof buf, "device watchdog: prefill workgroup %d waited too long at grid barrier %d (op %d, layer %d)",
             f.cta, f.pc, f.op, f.layer);
    return g.fail(MK_ETIMEOUT, buf);
  }
  return MK_OK;
}

int ctx_run(mk_ctx* c, int n, int first_token, const int32_t* forced, int32_t* tokens_out, float* logits_out) {
  Engine& g = c->g;
  const mk_config& k = c->cfg;
  const int pos0 = c->pos;
  if (n < 1) return g.fail(MK_EINVAL, "n_steps must be at least 1");
  if ((int64_t)pos0 + n > k.max_seq) return g.fail(MK_ERANGE, "decode would run past max_seq");
  HIPCHK(g, hipSetDevice(g.device));
  if (forced) {
    for (int i = 0; i < n; ++i)
      if (forced[i] < 0 || forced[i] >= k.vocab) return g.fail(MK_ERANGE, "token id outside [0, vocab)");
    HIPCHK(g, hipMemcpyAsync(g.d_forced, forced, n * sizeof(int32_t), hipMemcpyHostToDevice, g.stream));
  }
  if (logits_out && (int64_t)n * k.vocab > g.logits_cap) {
    if (g.d_logits) {
      HIPCHK(g, hipStreamSynchronize(g.stream));
      hipFree(g.d_logits);
      g.allocs.erase(std::remove(g.allocs.begin(), g.allocs.end(), (void*)g.d_logits), g.allocs.end());
      g.d_logits = nullptr;
    }
    CHK(g.alloc(&g.d_logits, (size_t)n * k.vocab * 4));
    g.logits_cap = (int64_t)n * k.vocab;
  }
  // re-arm every sync buffer and the KV positions this launch writes
  HIPCHK(g, mk_launch_fill32((uint32_t*)g.d_arena, g.lmp_word_off, kSent32, g.stream));
  HIPCHK(g, mk_launch_fill32((uint32_t*)g.d_arena + g.lmp_word_off, g.arena_words - g.lmp_word_off, 0u, g.stream));
  HIPCHK(g, mk_launch_fill_kv(c->d_kc, c->d_vc, (int64_t)k.n_layers * k.n_kv_heads, k.max_seq, k.head_dim, pos0, pos0 + n,
                              g.stream));
  KParams kp{};
  fill_common_params(g, kp);
  kp.n_steps = n;
  kp.pos0 = pos0;
  kp.first_token = first_token;
  kp.chain = 0;
  kp.forced = forced ? g.d_forced : nullptr;
  kp.tokens = g.d_tokens;
  kp.logits = logits_out ? g.d_logits : nullptr;
  kp.embed = c->d_embed;
  kp.norms = c->d_norms;
  kp.rope = c->d_rope;
  kp.kc = c->d_kc;
  kp.vc = c->d_vc;
  kp.xa = c->xa;
  kp.xm = c->xm;
  kp.q = c->q;
  kp.o = c->o;
  kp.m = c->m;
  kp.att_o = c->att_o;
  kp.att_ml = c->att_ml;
  kp.att_cnt = c->att_cnt;
  kp.lmp = c->lmp;
  kp.lmp_es = c->lmp_es;
  kp.lmp_rs = c->lmp_rs;
  kp.lmk = c->lmk;
  kp.lmk_es = c->lmk_es;
  kp.lmk_rs = c->lmk_rs;
  kp.top_k = c->top_k;
  c->last_top_k = c->top_k;
  kp.inv_temp = 1.0f / c->temperature;
  kp.seed_lo = (uint32_t)c->seed;
  kp.seed_hi = (uint32_t)(c->seed >> 32);
  kp.L = k.n_layers;
  kp.d = k.d_model;
  kp.nq = k.n_heads;
  kp.nkv = k.n_kv_heads;
  kp.hd = k.head_dim;
  kp.f = k.ffn;
  kp.V = k.vocab;
  kp.max_seq = k.max_seq;
  kp.eps = k.rms_eps;
  kp.vec_floats = (g.plan.lds_bytes - lds_bytes_for(0)) / 4;
  c->last_pos0 = pos0;
  c->last_n = n;
  int rc = launch(g, kp, n);
  // algorithmic bytes per step: the weights (the plan's figure already holds
  // the norm gains and one embedding row) + K/V of positions 0..pos
  const int64_t kv_pos = 2LL * k.n_layers * k.n_kv_heads * k.head_dim * 2;
  int64_t bytes = 0;
  for (int s = 0; s < n; ++s) bytes += g.plan.weight_bytes + kv_pos * (pos0 + s + 1);
  g.last.algo_bytes = bytes;
  g.last.kv_bytes_per_pos = kv_pos;
  g.last.pos0 = pos0;
  if (rc != MK_OK && rc != MK_ENAN) return rc;
  HIPCHK(g, hipMemcpy(tokens_out, g.d_tokens, n * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (logits_out) HIPCHK(g, hipMemcpy(logits_out, g.d_logits, (size_t)n * k.vocab * 4, hipMemcpyDeviceToHost));
  return rc;
}

void advance(mk_ctx* c, int n, const int32_t* consumed_first, const int32_t* forced, const int32_t* toks) {
  c->hist.resize(c->pos);
  for (int s = 0; s < n; ++s) c->hist.push_back(forced ? forced[s] : (s == 0 ? *consumed_first : toks[s - 1]));
  c->pos += n;
  c->next_tok = toks[n - 1];
}

}  // namespace

extern "C" {

int mk_default_options(mk_options* o) {
  if (!o) return MK_EINVAL;
  o->sync_mode = MK_SYNC_SENTINEL;
  o->xcd_replicas = 8;
  o->attn_splits = 0;
  o->trace_steps = 0;
  o->watchdog_us = 2000000;
  o->grid = 0;
  o->work_queue = 0;
  return MK_OK;
}

static mk::Dims dims_of(const mk_config* cfg) {
  mk::Dims d;
  d.L = cfg->n_layers;
  d.d = cfg->d_model;
  d.nq = cfg->n_heads;
  d.nkv = cfg->n_kv_heads;
  d.hd = cfg->head_dim;
  d.f = cfg->ffn;
  d.V = cfg->vocab;
  d.max_seq = cfg->max_seq;
  return d;
}

int mk_plan_check(const mk_config* cfg, const mk_options* opts, int32_t n_cta, mk_plan_info* info, const char** msg) {
  static thread_local std::string m;
  mk_options o;
  if (msg) *msg = "";
  if (!cfg || sanitize_options(opts, &o) != MK_OK) {
    m = "invalid options";
    if (msg) *msg = m.c_str();
    return MK_EINVAL;
  }
  Plan p;
  m = build_plan(dims_of(cfg), n_cta, o.attn_splits, o.xcd_replicas, o.sync_mode, &p);
  if (!m.empty()) {
    if (msg) *msg = m.c_str();
    return MK_EINVAL;
  }
  if (info) {
    info->n_cta = p.n_cta;
    info->max_ins_per_cta = p.max_ins;
    info->n_sync_ids = p.n_sync;
    info->lds_bytes = p.lds_bytes;
    info->stream_chunks = (int64_t)p.chunks.size();
    info->stream_bytes = p.stream_bytes();
    info->weight_bytes = p.weight_bytes;
    int mn = INT32_MAX, mx = 0;
    for (int32_t v : p.wave_n) {
      mn = std::min(mn, v);
      mx = std::max(mx, v);
    }
    info->min_wave_chunks = mn;
    info->max_wave_chunks = mx;
    info->attn_splits = p.S;
    info->specialised = fits_specialised(p) ? 1 : 0;
  }
  return MK_OK;
}

int mk_create(const mk_config* cfg, const mk_options* opts, int device, void* hip_stream, mk_ctx** out) {
  g_create_error.clear();
  if (!cfg || !out) {
    g_create_error = "NULL argument";
    return MK_EINVAL;
  }
  *out = nullptr;
  mk_ctx* c = new mk_ctx();
  c->cfg = *cfg;
  Engine& g = c->g;
  auto bail = [&](int rc) {
    g_create_error = g.err.empty() ? "mk_create failed" : g.err;
    g.release();
    delete c;
    return rc;
  };
  mk_options o;
  if (sanitize_options(opts, &o) != MK_OK) {
    g.err = "invalid options";
    return bail(MK_EINVAL);
  }
  // the grid depends on the occupancy, which depends on the LDS size: size it first
  int rc = engine_setup(g, device, hip_stream, &o, plan_lds_bytes(dims_of(cfg)));
  if (rc != MK_OK) return bail(rc);
  std::string msg = build_plan(dims_of(cfg), g.grid, o.attn_splits, o.xcd_replicas, o.sync_mode, &g.plan);
  if (!msg.empty()) {
    g.err = msg;
    return bail(MK_EINVAL);
  }
  if ((rc = upload_plan(g)) != MK_OK) return bail(rc);
  const mk_config& k = *cfg;
  const int64_t kv_words = (int64_t)k.n_layers * k.n_kv_heads * k.max_seq * k.head_dim;
  if ((rc = g.alloc(&c->d_kc, kv_words * 2)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&c->d_vc, kv_words * 2)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&c->d_embed, (size_t)k.vocab * k.d_model * 2)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&c->d_norms, (size_t)(2 * k.n_layers + 1) * k.d_model * 2)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&c->d_rope, (size_t)k.max_seq * k.head_dim * 4)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&g.d_tokens, (size_t)k.max_seq * 4)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&g.d_forced, (size_t)k.max_seq * 4)) != MK_OK) return bail(rc);
  if ((rc = ctx_alloc_arena(c)) != MK_OK) return bail(rc);
  if ((rc = ctx_alloc_prefill(c)) != MK_OK) return bail(rc);
  // RoPE table: cos/sin of pos * theta^(-2i/hd), computed in double
  {
    const int hh = k.head_dim / 2;
    std::vector<float> t((size_t)k.max_seq * hh * 2);
    for (int p = 0; p < k.max_seq; ++p)
      for (int i = 0; i < hh; ++i) {
        const double w = pow((double)k.rope_theta, -2.0 * i / k.head_dim);
        const double a = (double)p * w;
        t[((size_t)p * hh + i) * 2] = (float)cos(a);
        t[((size_t)p * hh + i) * 2 + 1] = (float)sin(a);
      }
    hipError_t e = hipMemcpy(c->d_rope, t.data(), t.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      g.hip_fail(e, "rope upload");
      return bail(MK_EHIP);
    }
  }
  *out = c;
  return MK_OK;
}

int mk_load_weights(mk_ctx* c, const mk_weights* w) {
  if (!c || !w) return MK_EINVAL;
  Engine& g = c->g;
  const mk_config& k = c->cfg;
  const int L = k.n_layers;
  if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
    return g.fail(MK_EINVAL, "a weight pointer is NULL");
  HIPCHK(g, hipSetDevice(g.device));
  std::vector<const uint16_t*> mats(7 * L + 1, nullptr);
  for (int l = 0; l < L; ++l) {
    mats[7 * l + MQ] = (const uint16_t*)w->wq[l];
    mats[7 * l + MK] = (const uint16_t*)w->wk[l];
    mats[7 * l + MV] = (const uint16_t*)w->wv[l];
    mats[7 * l + MO] = (const uint16_t*)w->wo[l];
    mats[7 * l + MG] = (const uint16_t*)w->w_gate[l];
    mats[7 * l + MU] = (const uint16_t*)w->w_up[l];
    mats[7 * l + MD] = (const uint16_t*)w->w_down[l];
  }
  mats[7 * L] = (const uint16_t*)w->lm_head;
  CHK(repack(g, mats));
  if (c->pf_ok) {
    // canonical copy for the prefill GEMMs: per layer [wq; wk; wv], wo, wg, wu, wd
    const int qd = k.n_heads * k.head_dim, kvd = k.n_kv_heads * k.head_dim;
    const size_t d = k.d_model, f = k.ffn;
    const size_t sz[7] = {qd * d, kvd * d, kvd * d, d * qd, f * d, f * d, d * f};
    uint16_t* dst = c->d_canon;
    for (int l = 0; l < L; ++l)
      for (int m = 0; m < 7; ++m) {
        HIPCHK(g, hipMemcpyAsync(dst, mats[7 * l + m], sz[m] * 2, hipMemcpyDeviceToDevice, g.stream));
        dst += sz[m];
      }
  }
  const size_t drow = (size_t)k.d_model * 2;
  HIPCHK(g, hipMemcpyAsync(c->d_embed, w->embed, (size_t)k.vocab * drow, hipMemcpyDeviceToDevice, g.stream));
  for (int l = 0; l < L; ++l) {
    if (!w->attn_norm[l] || !w->mlp_norm[l]) return g.fail(MK_EINVAL, "a norm pointer is NULL");
    HIPCHK(g, hipMemcpyAsync((uint8_t*)c->d_norms + (2 * l) * drow, w->attn_norm[l], drow, hipMemcpyDeviceToDevice, g.stream));
    HIPCHK(g, hipMemcpyAsync((uint8_t*)c->d_norms + (2 * l + 1) * drow, w->mlp_norm[l], drow, hipMemcpyDeviceToDevice, g.stream));
  }
  HIPCHK(g, hipMemcpyAsync((uint8_t*)c->d_norms + 2 * L * drow, w->final_norm, drow, hipMemcpyDeviceToDevice, g.stream));
  HIPCHK(g, hipStreamSynchronize(g.stream));
  c->state = ST_LOADED;
  c->pos = 0;
  c->hist.clear();
  return MK_OK;
}

int mk_prefill(mk_ctx* c, const int32_t* ids, int32_t n, int32_t* t0_out) {
  if (!c || !ids || !t0_out) return MK_EINVAL;
  if (c->state < ST_LOADED) return c->g.fail(MK_ESTATE, "prefill before mk_load_weights");
  if (n < 1) return c->g.fail(MK_EINVAL, "empty prompt");
  if (n > c->cfg.max_seq) return c->g.fail(MK_ERANGE, "prompt longer than max_seq");
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->cfg.vocab) return c->g.fail(MK_ERANGE, "token id outside [0, vocab)");
  c->pos = 0;
  c->hist.clear();
  c->g.last.prefill_ms = 0;
  c->g.last.prefill_positions = 0;
  c->g.last.prefill_grid = 0;
  // positions 0..n-2 on the MFMA prefill kernel (unless MK_PREFILL_STEPS asks for the
  // token-by-token path), then the last prompt token through the decode monokernel,
  // which chooses t0 exactly as every later step is chosen
  const bool mfma = c->pf_ok && n >= 2 && !getenv("MK_PREFILL_STEPS");
  const int head = mfma ? n - 1 : 0;
  int rc = MK_OK;
  if (mfma) {
    rc = ctx_prefill_mfma(c, ids, head);
    if (rc != MK_OK) {
      c->state = ST_LOADED;
      return rc;
    }
    c->pos = head;
    c->hist.assign(ids, ids + head);
  }
  const double pf_ms = c->g.last.prefill_ms;
  std::vector<int32_t> toks(n - head);
  rc = ctx_run(c, n - head, 0, ids + head, toks.data(), nullptr);
  c->g.last.prefill_ms = pf_ms;
  c->g.last.prefill_positions = head;
  c->g.last.prefill_grid = mfma ? c->pf_grid : 0;
  if (rc != MK_OK) {
    c->state = ST_LOADED;
    return rc;
  }
  advance(c, n - head, nullptr, ids + head, toks.data());
  *t0_out = toks[n - head - 1];
  c->state = ST_READY;
  return MK_OK;
}

int mk_decode(mk_ctx* c, int32_t n, int32_t* tokens_out, float* logits_out) {
  if (!c || !tokens_out) return MK_EINVAL;
  if (c->state < ST_READY) return c->g.fail(MK_ESTATE, "decode before prefill");
  const int first = c->next_tok;
  int rc = ctx_run(c, n, first, nullptr, tokens_out, logits_out);
  if (rc != MK_OK) {
    if (rc == MK_ETIMEOUT) c->state = ST_LOADED;
    return rc;
  }
  advance(c, n, &first, nullptr, tokens_out);
  return MK_OK;
}

int mk_decode_forced(mk_ctx* c, int32_t n, const int32_t* tokens_in, int32_t* tokens_out, float* logits_out) {
  if (!c || !tokens_in || !tokens_out) return MK_EINVAL;
  if (c->state < ST_READY) return c->g.fail(MK_ESTATE, "decode before prefill");
  int rc = ctx_run(c, n, 0, tokens_in, tokens_out, logits_out);
  if (rc != MK_OK) {
    if (rc == MK_ETIMEOUT) c->state = ST_LOADED;
    return rc;
  }
  advance(c, n, nullptr, tokens_in, tokens_out);
  return MK_OK;
}

int mk_generate(mk_ctx* c, const int32_t* ids, int32_t n_prompt, int32_t n_steps, int32_t* tokens_out) {
  if (!c || !tokens_out) return MK_EINVAL;
  int rc = mk_prefill(c, ids, n_prompt, tokens_out);
  if (rc != MK_OK || n_steps == 0) return rc;
  return mk_decode(c, n_steps, tokens_out + 1, nullptr);
}

const char* mk_kernel_name(const mk_ctx* c) {
  if (!c) return "";
  static const char* const names[4] = {"mk_monokernel", "mk_monokernel_w4h128", "mk_monokernel_w4h128_ctr",
                                       "mk_monokernel_w4h128_long"};
  const int kind = c->g.last_kind >= 0 ? c->g.last_kind : kernel_kind(c->g, c->pos);
  return names[kind];
}

int mk_set_sampling(mk_ctx* c, int32_t top_k, float temperature, uint64_t seed) {
  if (!c) return MK_EINVAL;
  if (top_k < 1 || top_k > kMaxTopK || top_k > c->cfg.vocab)
    return c->g.fail(MK_EINVAL, "top_k outside [1, min(16, vocab)]");
  if (top_k > 1 && !(temperature > 0.0f && temperature < INFINITY))
    return c->g.fail(MK_EINVAL, "temperature must be positive and finite");
  c->top_k = top_k;
  c->temperature = top_k > 1 ? temperature : 1.0f;
  c->seed = seed;
  return MK_OK;
}

int mk_rewind(mk_ctx* c, int32_t pos) {
  if (!c) return MK_EINVAL;
  if (c->state < ST_READY) return c->g.fail(MK_ESTATE, "rewind before prefill");
  if (pos < 1 || pos > c->pos) return c->g.fail(MK_ERANGE, "rewind position outside [1, current]");
  if (pos == c->pos) return MK_OK;
  c->next_tok = c->hist[pos];
  c->pos = pos;
  c->hist.resize(pos);
  return MK_OK;
}

int mk_position(const mk_ctx* c, int32_t* pos, int32_t* next_token) {
  if (!c) return MK_EINVAL;
  if (pos) *pos = c->pos;
  if (next_token) *next_token = c->next_tok;
  return MK_OK;
}

int mk_stats(const mk_ctx* c, mk_stats_t* out) {
  if (!c || !out) return MK_EINVAL;
  *out = c->g.last;
  return MK_OK;
}

int mk_count_sentinels(mk_ctx* c, int64_t* count) {
  if (!c || !count) return MK_EINVAL;
  Engine& g = c->g;
  if (c->last_n < 1) return g.fail(MK_ESTATE, "no launch yet");
  HIPCHK(g, hipSetDevice(g.device));
  unsigned long long* d = nullptr;
  HIPCHK(g, hipMalloc(&d, 8));
  hipError_t e = hipMemsetAsync(d, 0, 8, g.stream);
  const int el = (c->last_n - 1) % 3;
  for (const auto& r : c->epoch_regions[el])
    if (e == hipSuccess) e = mk_launch_count32((const uint32_t*)g.d_arena + r.off, r.words, kSent32, d, g.stream);
  const mk_config& k = c->cfg;
  if (e == hipSuccess)
    e = mk_launch_count_kv(c->d_kc, c->d_vc, (int64_t)k.n_layers * k.n_kv_heads, k.max_seq, k.head_dim, c->last_pos0,
                           c->last_pos0 + c->last_n, d, g.stream);
  unsigned long long h = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&h, d, 8, hipMemcpyDeviceToHost, g.stream);
  if (e == hipSuccess) e = hipStreamSynchronize(g.stream);
  // argmax keys of the last step (sentinel 0)
  std::vector<uint64_t> keys(c->lmp_es);
  if (e == hipSuccess)
    e = hipMemcpy(keys.data(), c->lmp + el * c->lmp_es, keys.size() * 8, hipMemcpyDeviceToHost);
  hipFree(d);
  if (e != hipSuccess) return g.hip_fail(e, "sentinel count");
  for (uint64_t v : keys) h += v == kSent64;
  if (c->last_top_k > 1) {
    // the top-k lists of the last step: [R][lm_slots][kMaxTopK], the first top_k of each written
    std::vector<uint64_t> lists(c->lmk_es);
    e = hipMemcpy(lists.data(), c->lmk + el * c->lmk_es, lists.size() * 8, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return g.hip_fail(e, "sentinel count");
    for (int64_t i = 0; i < c->lmk_es; ++i) h += (i % kMaxTopK) < c->last_top_k && lists[i] == kSent64;
  }
  *count = (int64_t)h;
  return MK_OK;
}

int mk_count_sentinels_noalloc(mk_ctx* c, int64_t* count) {
  if (!c || !count) return MK_EINVAL;
  Engine& g = c->g;
  if (c->last_n < 1) return g.fail(MK_ESTATE, "no launch yet");
  HIPCHK(g, hipSetDevice(g.device));
  void* sp = nullptr;
  size_t sbytes = 0;
  HIPCHK(g, mk_scratch_address(g.device, &sp, &sbytes));
  if (sbytes < sizeof(unsigned long long)) return g.fail(MK_EINVAL, "the static scratch is smaller than one counter");
  unsigned long long* d = (unsigned long long*)sp;
  // cleared by a fill kernel (no memset node), then the same counts as mk_count_sentinels,
  // the argmax keys and top-k lists counted on the device as well
  hipError_t e = mk_launch_fill32((uint32_t*)d, 2, 0u, g.stream);
  const int el = (c->last_n - 1) % 3;
  for (const auto& r : c->epoch_regions[el])
    if (e == hipSuccess) e = mk_launch_count32((const uint32_t*)g.d_arena + r.off, r.words, kSent32, d, g.stream);
  const mk_config& k = c->cfg;
  if (e == hipSuccess)
    e = mk_launch_count_kv(c->d_kc, c->d_vc, (int64_t)k.n_layers * k.n_kv_heads, k.max_seq, k.head_dim, c->last_pos0,
                           c->last_pos0 + c->last_n, d, g.stream);
  if (e == hipSuccess) e = mk_launch_count64(c->lmp + el * c->lmp_es, c->lmp_es, 1, 1, kSent64, d, g.stream);
  if (e == hipSuccess && c->last_top_k > 1)
    e = mk_launch_count64(c->lmk + el * c->lmk_es, c->lmk_es, kMaxTopK, c->last_top_k, kSent64, d, g.stream);
  unsigned long long h = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&h, d, sizeof h, hipMemcpyDeviceToHost, g.stream);
  if (e == hipSuccess) e = hipStreamSynchronize(g.stream);
  if (e != hipSuccess) return g.hip_fail(e, "sentinel count");
  *count = (int64_t)h;
  return MK_OK;
}

int mk_read_trace(mk_ctx* c, uint32_t* host_buf, int64_t capacity, int64_t* n_records) {
  if (!c || !n_records) return MK_EINVAL;
  Engine& g = c->g;
  *n_records = g.trace_words / 8;
  if (!host_buf) return MK_OK;
  if (capacity < *n_records) return g.fail(MK_EINVAL, "trace buffer too small");
  if (g.trace_words) HIPCHK(g, hipMemcpy(host_buf, g.d_trace, g.trace_words * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_debug_streams(const mk_ctx* c, const void** base, const void** wave_off, const void** wave_n) {
  if (!c || !base || !wave_off || !wave_n) return MK_EINVAL;
  *base = c->g.d_stream;
  *wave_off = c->g.d_wave_off;
  *wave_n = c->g.d_wave_n;
  return MK_OK;
}

int mk_debug_layout(const mk_ctx* c, int64_t* offsets) {
  if (!c || !offsets) return MK_EINVAL;
  for (int i = 0; i < 16; ++i) offsets[i] = c->layout[i];
  return MK_OK;
}

int mk_debug_arena(mk_ctx* c, int64_t word_off, int64_t n_words, uint32_t* host) {
  if (!c || !host || word_off < 0 || n_words < 0 || word_off + n_words > c->g.arena_words) return MK_EINVAL;
  HIPCHK(c->g, hipMemcpy(host, (uint32_t*)c->g.d_arena + word_off, n_words * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_debug_kv(mk_ctx* c, int32_t layer, int32_t kv_head, int32_t pos0, int32_t n, uint16_t* k_out, uint16_t* v_out) {
  if (!c || !k_out || !v_out) return MK_EINVAL;
  const mk_config& k = c->cfg;
  if (layer < 0 || layer >= k.n_layers || kv_head < 0 || kv_head >= k.n_kv_heads || pos0 < 0 || n < 0 ||
      (int64_t)pos0 + n > k.max_seq)
    return c->g.fail(MK_EINVAL, "KV range outside the cache");
  HIPCHK(c->g, hipSetDevice(c->g.device));
  const int64_t off = (((int64_t)layer * k.n_kv_heads + kv_head) * k.max_seq + pos0) * k.head_dim;
  const size_t bytes = (size_t)n * k.head_dim * 2;
  HIPCHK(c->g, hipMemcpy(k_out, c->d_kc + off, bytes, hipMemcpyDeviceToHost));
  HIPCHK(c->g, hipMemcpy(v_out, c->d_vc + off, bytes, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_debug_prefill_marks(mk_ctx* c, uint64_t* host, int32_t capacity) {
  if (!c || !host) return MK_EINVAL;
  const int n = 5 * c->cfg.n_layers + 1;
  if (capacity < n) return c->g.fail(MK_EINVAL, "capacity below 1 + 5 n_layers");
  if (!c->d_pmarks) return c->g.fail(MK_ESTATE, "this context has no prefill kernel");
  HIPCHK(c->g, hipMemcpy(host, c->d_pmarks, (size_t)n * 8, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_debug_force_stall(mk_ctx* c, int32_t cta) {
  if (!c) return MK_EINVAL;
  if (cta < 0 || cta >= c->g.grid) return c->g.fail(MK_EINVAL, "no such workgroup");
  if (c->g.plan.sync_mode != MK_SYNC_SENTINEL) return c->g.fail(MK_EINVAL, "the stall test needs sentinel sync");
  c->g.stall_cta = cta;
  return MK_OK;
}

int mk_debug_progress(mk_ctx* c, uint32_t* host, int32_t capacity) {
  if (!c || !host || capacity < c->g.grid) return MK_EINVAL;
  HIPCHK(c->g, hipMemcpy(host, c->g.d_progress, (size_t)c->g.grid * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

const char* mk_last_error(const mk_ctx* c) {
  if (!c) return g_create_error.c_str();
  return c->g.err.c_str();
}

void mk_destroy(mk_ctx* c) {
  if (!c) return;
  hipSetDevice(c->g.device);
  c->g.release();
  delete c;
}

}  // extern "C"

// ============================================================ chain microbenchmark
struct mk_chain {
  Engine g;
  int n = 0, stages = 0;
  Buf y{};
};

extern "C" {

int mk_chain_create(int32_t n, int32_t stages, const void* W, const mk_options* opts, int device, void* hip_stream,
                    mk_chain** out) {
  g_create_error.clear();
  if (!out || !W) {
    g_create_error = "NULL argument";
    return MK_EINVAL;
  }
  *out = nullptr;
  mk_chain* ch = new mk_chain();
  Engine& g = ch->g;
  auto bail = [&](int rc) {
    g_create_error = g.err.empty() ? "mk_chain_create failed" : g.err;
    g.release();
    delete ch;
    return rc;
  };
  mk_options o;
  if (sanitize_options(opts, &o) != MK_OK) {
    g.err = "invalid options";
    return bail(MK_EINVAL);
  }
  mk::Dims dm;
  dm.chain = true;
  dm.chain_n = n;
  dm.chain_stages = stages;
  int rc = engine_setup(g, device, hip_stream, &o, plan_lds_bytes(dm));
  if (rc != MK_OK) return bail(rc);
  std::string msg = build_plan(dm, g.grid, 1, o.xcd_replicas, o.sync_mode, &g.plan);
  if (!msg.empty()) {
    g.err = msg;
    return bail(MK_EINVAL);
  }
  if ((rc = upload_plan(g)) != MK_OK) return bail(rc);
  ch->n = n;
  ch->stages = stages;
  const int R = g.plan.R;
  ch->y.rs = R > 1 ? n : 0;
  ch->y.ls = (int64_t)n * R;
  ch->y.es = 0;
  g.arena_words = ch->y.ls * stages;
  g.lmp_word_off = g.arena_words;
  if ((rc = g.alloc(&g.d_arena, g.arena_words * 4)) != MK_OK) return bail(rc);
  if ((rc = g.alloc(&g.d_tokens, 64)) != MK_OK) return bail(rc);
  ch->y.p = g.d_arena;
  std::vector<const uint16_t*> mats(stages);
  for (int i = 0; i < stages; ++i) mats[i] = (const uint16_t*)W + (int64_t)i * n * n;
  if ((rc = repack(g, mats)) != MK_OK) return bail(rc);
  *out = ch;
  return MK_OK;
}

int mk_chain_run(mk_chain* ch, const float* x0, float* y) {
  if (!ch || !x0 || !y) return MK_EINVAL;
  Engine& g = ch->g;
  HIPCHK(g, hipSetDevice(g.device));
  HIPCHK(g, mk_launch_fill32((uint32_t*)g.d_arena, g.arena_words, kSent32, g.stream));
  KParams kp{};
  fill_common_params(g, kp);
  kp.n_steps = 1;
  kp.chain = 1;
  kp.tokens = g.d_tokens;
  kp.y = ch->y;
  kp.x0 = x0;
  kp.chain_n = ch->n;
  kp.L = ch->stages;
  kp.vec_floats = (g.plan.lds_bytes - lds_bytes_for(0)) / 4;
  int rc = launch(g, kp, 1);
  g.last.algo_bytes = g.plan.weight_bytes;
  if (rc != MK_OK) return rc;
  // y[i] = replica 0 of stage i
  HIPCHK(g, hipMemcpy2DAsync(y, (size_t)ch->n * 4, ch->y.p, (size_t)ch->y.ls * 4, (size_t)ch->n * 4, ch->stages,
                             hipMemcpyDeviceToDevice, g.stream));
  HIPCHK(g, hipStreamSynchronize(g.stream));
  return MK_OK;
}

int mk_chain_read_trace(mk_chain* ch, uint32_t* host_buf, int64_t capacity, int64_t* n_records) {
  if (!ch || !n_records) return MK_EINVAL;
  Engine& g = ch->g;
  *n_records = g.trace_words / 8;
  if (!host_buf) return MK_OK;
  if (capacity < *n_records) return g.fail(MK_EINVAL, "trace buffer too small");
  if (g.trace_words) HIPCHK(g, hipMemcpy(host_buf, g.d_trace, g.trace_words * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_debug_ts(mk_ctx* c, uint64_t* host, int64_t capacity) {
  if (!c || !host) return MK_EINVAL;
  Engine& g = c->g;
  const int64_t n = (int64_t)g.grid * g.plan.max_ins * 8;
  if (capacity < n) return MK_EINVAL;
  HIPCHK(g, hipMemcpy(host, g.d_ts, n * 8, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_chain_debug_ts(mk_chain* ch, uint64_t* host, int64_t capacity) {
  if (!ch || !host) return MK_EINVAL;
  Engine& g = ch->g;
  const int64_t n = (int64_t)g.grid * g.plan.max_ins * 8;
  if (capacity < n) return MK_EINVAL;
  HIPCHK(g, hipMemcpy(host, g.d_ts, n * 8, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_chain_stats(const mk_chain* ch, mk_stats_t* out) {
  if (!ch || !out) return MK_EINVAL;
  *out = ch->g.last;
  return MK_OK;
}

const char* mk_chain_last_error(const mk_chain* ch) {
  if (!ch) return g_create_error.c_str();
  return ch->g.err.c_str();
}

void mk_chain_destroy(mk_chain* ch) {
  if (!ch) return;
  hipSetDevice(ch->g.device);
  ch->g.release();
  delete ch;
}

}  // extern "C"

// ============================================================ calibration probes
namespace {

int probe_fail(int rc, const char* what, hipError_t e = hipSuccess) {
  g_create_error = what;
  if (e != hipSuccess) {
    g_create_error += ": ";
    g_create_error += hipGetErrorString(e);
  }
  return rc;
}

#define PROBE_HIP(call, what)                          \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return probe_fail(MK_EHIP, what, e_); \
  } while (0)

}  // namespace

extern "C" {

int mk_probe_launch(int device, void* hip_stream, int32_t n_launches, double* us_pipelined, double* us_round_trip) {
  if (n_launches < 1 || !us_pipelined || !us_round_trip) return probe_fail(MK_EINVAL, "bad probe arguments");
  g_create_error.clear();
  hipStream_t s = (hipStream_t)hip_stream;
  PROBE_HIP(hipSetDevice(device), "hipSetDevice");
  PROBE_HIP(mk_launch_probe_empty(s), "empty launch");
  PROBE_HIP(hipStreamSynchronize(s), "sync");
  auto now = [] { return std::chrono::steady_clock::now(); };
  auto t0 = now();
  for (int i = 0; i < n_launches; ++i) PROBE_HIP(mk_launch_probe_empty(s), "empty launch");
  PROBE_HIP(hipStreamSynchronize(s), "sync");
  auto t1 = now();
  for (int i = 0; i < n_launches; ++i) {
    PROBE_HIP(mk_launch_probe_empty(s), "empty launch");
    PROBE_HIP(hipStreamSynchronize(s), "sync");
  }
  auto t2 = now();
  *us_pipelined = std::chrono::duration<double, std::micro>(t1 - t0).count() / n_launches;
  *us_round_trip = std::chrono::duration<double, std::micro>(t2 - t1).count() / n_launches;
  return MK_OK;
}

int mk_probe_read(int device, void* hip_stream, const void* buf, int64_t bytes, int32_t repeats, double* gb_per_s) {
  if (!buf || bytes < 16 || bytes % 16 || ((uintptr_t)buf & 15) || repeats < 1 || !gb_per_s)
    return probe_fail(MK_EINVAL, "bad probe arguments");
  g_create_error.clear();
  hipStream_t s = (hipStream_t)hip_stream;
  PROBE_HIP(hipSetDevice(device), "hipSetDevice");
  hipDeviceProp_t prop;
  PROBE_HIP(hipGetDeviceProperties(&prop, device), "device properties");
  const int grid = prop.multiProcessorCount * 2;  // two workgroups of 512 threads per CU
  void* sink = nullptr;
  PROBE_HIP(hipMalloc(&sink, (size_t)grid * 512 * 16), "sink allocation");
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = mk_launch_probe_read(buf, bytes / 16, sink, grid, s);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(a, s);
  for (int i = 0; i < repeats && e == hipSuccess; ++i) e = mk_launch_probe_read(buf, bytes / 16, sink, grid, s);
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) hipEventDestroy(a);
  if (b) hipEventDestroy(b);
  hipFree(sink);
  if (e != hipSuccess) return probe_fail(MK_EHIP, "read probe", e);
  *gb_per_s = (double)bytes * repeats / (ms * 1e-3) / 1e9;
  return MK_OK;
}

int mk_probe_barrier(int device, void* hip_stream, int32_t rounds, double* us_per_barrier) {
  if (rounds < 1 || rounds > 1000000 || !us_per_barrier) return probe_fail(MK_EINVAL, "bad probe arguments");
  g_create_error.clear();
  hipStream_t s = (hipStream_t)hip_stream;
  PROBE_HIP(hipSetDevice(device), "hipSetDevice");
  hipDeviceProp_t prop;
  PROBE_HIP(hipGetDeviceProperties(&prop, device), "device properties");
  int occ = 0;
  PROBE_HIP(mk_probe_barrier_occupancy(&occ), "occupancy");
  const int grid = prop.multiProcessorCount;  // one workgroup per CU, all resident
  if (occ < 1) return probe_fail(MK_EOCC, "barrier probe does not fit a CU");
  uint32_t* counter = nullptr;
  uint64_t* out = nullptr;
  PROBE_HIP(hipMalloc(&counter, 4), "counter allocation");
  hipError_t e = hipMalloc(&out, 16);
  if (e == hipSuccess) e = mk_launch_fill32(counter, 1, 0u, s);
  if (e == hipSuccess) e = mk_launch_fill32((uint32_t*)out, 4, 0u, s);
  if (e == hipSuccess) e = mk_launch_probe_barrier(counter, rounds, 100000000ull /* 1 s */, out, grid, s);
  uint64_t h[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpyAsync(h, out, 16, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipFree(counter);
  if (out) hipFree(out);
  if (e != hipSuccess) return probe_fail(MK_EHIP, "barrier probe", e);
  if (h[1]) return probe_fail(MK_ETIMEOUT, "a barrier round did not complete within 1 s");
  *us_per_barrier = (double)h[0] * 0.01 / rounds;  // 100 MHz device clock
  return MK_OK;
}

int mk_probe_handoff(int device, void* hip_stream, int32_t mode, int32_t same_xcd, int32_t rounds, double* us_handoff,
                     double* stream_gb_per_s, double* same_xcd_fraction) {
  if (mode < 0 || mode > 3 || rounds < 1 || rounds > 100000 || !us_handoff || !stream_gb_per_s || !same_xcd_fraction)
    return probe_fail(MK_EINVAL, "bad probe arguments");
  g_create_error.clear();
  hipStream_t s = (hipStream_t)hip_stream;
  PROBE_HIP(hipSetDevice(device), "hipSetDevice");
  hipDeviceProp_t prop;
  PROBE_HIP(hipGetDeviceProperties(&prop, device), "device properties");
  const int grid = prop.multiProcessorCount, pairs = mk_probe_handoff_pairs();
  int occ = 0;
  PROBE_HIP(mk_probe_handoff_occupancy(&occ), "occupancy");
  if (occ < 1) return probe_fail(MK_EOCC, "handoff probe does not fit a CU");
  if (grid < 2 * pairs) return probe_fail(MK_EOCC, "handoff probe needs 32 CUs");
  const int64_t buf_bytes = 1LL << 30;
  const int stream_chunks = 24000;
  void *buf = nullptr, *sink = nullptr;
  uint32_t* words = nullptr;  // flags [pairs][2][64], then timeouts
  uint64_t* ticks = nullptr;
  int32_t* xcc = nullptr;
  const int64_t n_words = (int64_t)pairs * 2 * 64 + 1;
  hipError_t e = hipMalloc(&buf, buf_bytes);
  if (e == hipSuccess) e = hipMalloc(&sink, (size_t)grid * 512 * 16);
  if (e == hipSuccess) e = hipMalloc((void**)&words, n_words * 4);
  if (e == hipSuccess) e = hipMalloc((void**)&ticks, pairs * 8);
  if (e == hipSuccess) e = hipMalloc((void**)&xcc, pairs * 2 * 4);
  if (e == hipSuccess) e = mk_launch_fill32(words, n_words, 0u, s);
  if (e == hipSuccess) e = mk_launch_fill32((uint32_t*)ticks, pairs * 2, 0u, s);
  if (e == hipSuccess) e = mk_launch_fill32((uint32_t*)xcc, pairs * 2, 0xFFFFFFFFu, s);
  hipEvent_t a = nullptr, b = nullptr;
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipEventRecord(a, s);
  if (e == hipSuccess)
    e = mk_launch_probe_handoff(buf, (uint32_t)(buf_bytes / 1024), mode, same_xcd ? 1 : 0, rounds, stream_chunks, words,
                                ticks, xcc, words + n_words - 1, sink, grid, s);
  if (e == hipSuccess) e = hipEventRecord(b, s);
  std::vector<uint64_t> h_ticks(pairs);
  std::vector<int32_t> h_xcc(pairs * 2);
  uint32_t h_timeouts = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(h_ticks.data(), ticks, pairs * 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(h_xcc.data(), xcc, pairs * 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&h_timeouts, words + n_words - 1, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) hipEventDestroy(a);
  if (b) hipEventDestroy(b);
  hipFree(buf);
  hipFree(sink);
  hipFree(words);
  hipFree(ticks);
  hipFree(xcc);
  if (e != hipSuccess) return probe_fail(MK_EHIP, "handoff probe", e);
  if (h_timeouts) return probe_fail(MK_ETIMEOUT, "a handoff of the probe hit its spin limit");
  std::sort(h_ticks.begin(), h_ticks.end());
  *us_handoff = (double)h_ticks[pairs / 2] * 0.01 / rounds / 2.0;  // median pair, 100 MHz clock, half a round trip
  int same = 0;
  for (int i = 0; i < pairs; ++i) same += h_xcc[2 * i] == h_xcc[2 * i + 1];
  *same_xcd_fraction = (double)same / pairs;
  const double waves = mode == 1 ? grid * 7.0 : mode == 2 ? grid * 8.0 - pairs * 2 : mode == 3 ? (grid - 2.0 * pairs) * 8 : 0.0;
  *stream_gb_per_s = waves * stream_chunks * 1024.0 / (ms * 1e-3) / 1e9;
  return MK_OK;
}

}  // extern "C"
