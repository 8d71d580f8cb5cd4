/*
 * mk_diag.h -- diagnostics and calibration probes of the decode monokernel
 * library (include/mk.h holds the decoding calls).
 *
 * These calls read back what the product calls leave behind (sentinel counts,
 * the per-instruction time journal, the sync-buffer arena, fine per-op marks)
 * or run stand-alone calibration kernels.  "8 - Ecrire son megakernel"
 * (section 8.7) asks for exactly these aids when a megakernel is debugged: a
 * trace of every instruction's start and end and a record of where each
 * workgroup stood.  Conventions are those of mk.h: MK_OK or a negative code,
 * host buffers owned by the caller, the context's stream synchronised before
 * returning.
 */
#ifndef MK_DIAG_H
#define MK_DIAG_H

#include "mk.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Count words still holding a sentinel in the sync buffers of the last step
 * of the last launch and in the KV cache positions it wrote.  0 after a good run. */
int mk_count_sentinels(mk_ctx* ctx, int64_t* count);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the count of
 * mk_count_sentinels with no allocation.  Its counter lives in a static
 * device array of 256 bytes per GPU (held until the process ends) instead of
 * the 8 bytes mk_count_sentinels allocates per call; the array is found once
 * per device and reused, and cleared by a fill kernel at every call.  The
 * scratch does not grow with the model (one counter whatever the arena size),
 * so no size is refused.  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (other threads, other streams) race on the
 * counter.  Synchronises the context's stream; errors as mk_count_sentinels. */
int mk_count_sentinels_noalloc(mk_ctx* ctx, int64_t* count);

/* Copy the time journal of the last launch into host memory.  Each record is
 * 8 uint32: {cta, step, pc, op | layer << 8 | xcc << 24 | 1 << 31, t_wait_lo,
 * t_ready - t_wait, t_done - t_wait, t_pub - t_wait}, in ticks of the 100 MHz
 * device wall clock: t_ready = inputs staged, t_pub = the instruction's output
 * stores issued, t_done = after the workgroup's failure vote.  Unused records
 * are zero.  *n_records receives the record count (capacity query if
 * host_buf is NULL). */
int mk_read_trace(mk_ctx* ctx, uint32_t* host_buf, int64_t capacity_records, int64_t* n_records);

/* Diagnostics.  Copy n_words 32-bit words of the sync-buffer arena starting
 * at word_off into host memory.  mk_debug_layout gives the word offsets of
 * its regions: [0] xa, [1] xm, [2] q, [3] o, [4] m, [5] att_o, [6] att_ml,
 * [7] argmax keys (uint64), [8] arena size, [9] attention merge counters
 * (uint32 [n_layers][n_kv_heads]), [10] per-workgroup top-k keys of sampling
 * (uint64 [3][replicas][workgroups][16]). */
int mk_debug_layout(const mk_ctx* ctx, int64_t* offsets /* [16] */);
int mk_debug_arena(mk_ctx* ctx, int64_t word_off, int64_t n_words, uint32_t* host);
/* (step << 16) | (pc + 1) of the last instruction each workgroup finished in
 * the last launch; host receives `grid` words. */
int mk_debug_progress(mk_ctx* ctx, uint32_t* host, int32_t capacity);

/* Copy the cached K and V rows of positions [pos0, pos0 + n) of one layer and
 * kv head into host memory (fp16 bit patterns, [n][head_dim] each).
 * MK_EINVAL for a range outside the cache. */
int mk_debug_kv(mk_ctx* ctx, int32_t layer, int32_t kv_head, int32_t pos0, int32_t n, uint16_t* k_out, uint16_t* v_out);

/* Device-clock (100 MHz) times at which workgroup 0 left each grid barrier of
 * the last MFMA prefill launch: [0] the embedding stage, then per layer the
 * QKV, attention, O-projection, up/gate and down stages (1 + 5 n_layers
 * values; differences are stage durations).  MK_ESTATE when the context has
 * no prefill kernel. */
int mk_debug_prefill_marks(mk_ctx* ctx, uint64_t* host, int32_t capacity);

/* Failure-path test: in the next launch only, workgroup `cta` waits in step 0,
 * before its argmax, for a sync word the host never writes, so that wait's
 * watchdog fires ("8 - Ecrire son megakernel", section 8.7: a watchdog that
 * turns a lost dependency into a report) after the context's watchdog_us, the
 * fault record names that workgroup, and every other workgroup leaves its
 * own waits through the abort flag: the launch ends normally and returns
 * MK_ETIMEOUT.  Sentinel sync only (MK_EINVAL otherwise, or for a workgroup
 * outside the grid). */
int mk_debug_force_stall(mk_ctx* ctx, int32_t cta);

/* Device addresses of the repacked weight streams: base, per-wavefront chunk
 * offsets [grid * 8] (int64) and chunk counts [grid * 8] (int32). */
int mk_debug_streams(const mk_ctx* ctx, const void** base, const void** wave_off, const void** wave_n);

/* Fine timestamps of step 0 of the last launch (recorded only when the
 * environment variable MK_DEBUG_TS is set at run time): per workgroup and
 * instruction, 8 uint64 device-clock (100 MHz) marks taken by thread 0
 * (wavefront 0) {0 instruction start, 1 inputs polled, 2 inputs staged (after
 * the barrier), 3 op end, 4 failure check done, 5 GEMV: activations in
 * registers / short attention split: the wavefront's positions done / long
 * split: the first K/V group loaded (in LDS, or the first register batch
 * issued), 6 GEMV: the wavefront's own rows done / attention: split partials
 * published, 7 GEMV: first weight chunk read / short split: wavefront
 * partials combined / long split: the wavefront's positions done}; zero
 * where not recorded.  capacity is in uint64 and must be at least
 * grid * max_ins_per_cta * 8. */
int mk_debug_ts(mk_ctx* ctx, uint64_t* host, int64_t capacity);

/* Time journal of the last chain run (same record format as mk_read_trace). */
int mk_chain_read_trace(mk_chain* ch, uint32_t* host_buf, int64_t capacity_records, int64_t* n_records);
/* Fine timestamps of step 0 of the last chain run (layout of mk_debug_ts). */
int mk_chain_debug_ts(mk_chain* ch, uint64_t* host, int64_t capacity);

/* Calibration probes: the launch cost, the practical HBM read ceiling and the naive grid
 * barrier that "7 - AMD et le monokernel" (section 7.3) compares the NaN sentinel against.
 * Each runs on `hip_stream` of `device` and synchronises; errors: MK_EINVAL (arguments), MK_EHIP (HIP failure), MK_EOCC, MK_ETIMEOUT;
 * text from mk_last_error(NULL).
 * mk_probe_launch: n_launches empty-kernel launches back to back then one synchronisation
 *   (host microseconds per launch -> *us_pipelined), and n_launches launch + synchronise
 *   pairs (-> *us_round_trip).
 * mk_probe_read: reads `bytes` (a multiple of 16, 16-byte aligned device buffer, borrowed)
 *   `repeats` times with nontemporal 16-byte loads, two workgroups of 512 threads per CU, each
 *   wavefront reading 16 consecutive KB per round; GB/s from HIP events (one untimed warm-up
 *   pass first).
 * mk_probe_barrier: `rounds` (1..1e6) grid barriers of one workgroup per CU, each a release,
 *   an atomic add to one counter and system-scope polls until every workgroup has arrived;
 *   microseconds per barrier on the device clock.  A round that does not complete within 1 s
 *   ends every wait and returns MK_ETIMEOUT.
 * mk_probe_handoff: the latency of one cross-workgroup handoff (a system-scope store seen by
 *   a system-scope poll, "7 - AMD et le monokernel", section 7.3) while the chip streams 1 KB
 *   weight chunks through per-wavefront LDS rings (12 slots, nontemporal), one workgroup per
 *   CU, 16 workgroup pairs ping-ponging `rounds` (1..1e5) times.  mode 0: nothing streams;
 *   1: every CU streams on 7 wavefronts and the pairs' 8th wavefront only polls; 2: all 8
 *   wavefronts stream and the pairs' 8th consumes 4 chunks of its ring before each handoff;
 *   3: the pairs' CUs stream nothing and every other CU streams on 8 wavefronts.  same_xcd
 *   pairs workgroups k and k+8 (one XCD under round-robin dispatch), else 2k and 2k+1.
 *   Outputs: median microseconds per handoff (half a round trip), GB/s streamed over the
 *   launch, and the fraction of pairs whose two members reported the same XCC_ID.  Allocates
 *   and frees 1 GiB of device memory; a wait beyond its spin limit returns MK_ETIMEOUT. */
int mk_probe_launch(int device, void* hip_stream, int32_t n_launches, double* us_pipelined, double* us_round_trip);
int mk_probe_read(int device, void* hip_stream, const void* buf, int64_t bytes, int32_t repeats, double* gb_per_s);
int mk_probe_barrier(int device, void* hip_stream, int32_t rounds, double* us_per_barrier);
int mk_probe_handoff(int device, void* hip_stream, int32_t mode, int32_t same_xcd, int32_t rounds, double* us_handoff,
                     double* stream_gb_per_s, double* same_xcd_fraction);

#ifdef __cplusplus
}
#endif
#endif /* MK_DIAG_H */
