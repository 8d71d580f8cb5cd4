/*
 * mk.h -- C ABI of the batch-1 decode monokernel for MI355X (gfx950).
 *
 * One persistent GPU launch runs whole decode steps of a Llama-style fp16
 * decoder: RMSNorm + QKV + RoPE, split attention over an fp16 KV cache, the
 * attention reduction, O-projection, SwiGLU MLP, LM head and greedy argmax.
 * The method is the "monokernel" of "7 - AMD et le monokernel" (section 7.1:
 * one persistent kernel runs prefill, decode and sampling without
 * interruption) with the per-SM instruction interpreter of "8 - Ecrire son
 * megakernel" (section 8.2) and its one-wave launch (section 8.3).  Stages
 * synchronise through NaN sentinels written into the output buffers
 * ("7 - AMD et le monokernel", section 7.3); atomic counters
 * ("8 - Ecrire son megakernel", section 8.5) are kept as a comparison path.
 *
 * Conventions for every call:
 *  - returns MK_OK (0) or a negative MK_E* code; mk_last_error() gives text;
 *  - no call allocates or frees memory owned by the caller;
 *  - "device" pointers are addresses in the memory of the context's GPU
 *    (e.g. the data pointer of a torch CUDA tensor); "host" pointers are
 *    ordinary CPU memory owned by the caller;
 *  - work is enqueued on the HIP stream given at creation; calls that return
 *    results synchronise that stream before returning;
 *  - one context must not be used from two threads at once.
 *
 * Weight layout: fp16, row-major [out, in] ("a row is one dot product").
 * embed and lm_head are [vocab, d_model]; wq [n_heads*head_dim, d_model];
 * wk, wv [n_kv_heads*head_dim, d_model]; wo [d_model, n_heads*head_dim];
 * w_gate, w_up [ffn, d_model]; w_down [d_model, ffn]; norm gains [d_model].
 * RoPE rotates the pairs (i, i + head_dim/2) of each q and k head by the
 * angle pos * rope_theta^(-2i/head_dim); positions are 0-based.  Query head j
 * reads kv head floor(j * n_kv_heads / n_heads).
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MK_OK = 0,
  MK_EINVAL = -1,   /* bad argument or unsupported shape */
  MK_ENOMEM = -2,   /* a device or host allocation failed */
  MK_EHIP = -3,     /* a HIP runtime call failed */
  MK_ESTATE = -4,   /* call out of order (e.g. decode before prefill or before weights) */
  MK_ERANGE = -5,   /* position would run past max_seq, or a token id outside [0, vocab) */
  MK_EOCC = -6,     /* the kernel does not fit one wave of co-resident workgroups */
  MK_ETIMEOUT = -7, /* the device watchdog fired: a dependency was never satisfied */
  MK_ENAN = -8      /* a NaN logit was produced */
};

enum { MK_SYNC_SENTINEL = 0, MK_SYNC_COUNTER = 1 };

/* Decoder dimensions.  Constraints: head_dim in {64, 128, 256}; n_heads a
 * multiple of n_kv_heads; d_model, ffn multiples of 4; d_model, ffn,
 * n_heads*head_dim at most 16384; max_seq >= 2. */
typedef struct mk_config {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn, vocab, max_seq;
  float rms_eps, rope_theta;
} mk_config;

/* Run-time options (mk_default_options fills the defaults). */
typedef struct mk_options {
  int32_t sync_mode;     /* MK_SYNC_SENTINEL (default) or MK_SYNC_COUNTER */
  int32_t xcd_replicas;  /* copies of re-read activation vectors: 1, 2, 4 or 8 (default 8) */
  int32_t attn_splits;   /* sequence splits per kv head, 1..64 (0 = choose) */
  int32_t trace_steps;   /* record a per-instruction time journal for the first N steps (0 = off) */
  int32_t watchdog_us;   /* per-wait timeout inside the kernel, microseconds (default 2000000) */
  int32_t grid;          /* workgroups to launch (0 = CUs x occupancy; larger values are refused) */
  int32_t work_queue;    /* prefill work distribution: 0 = static deal of tiles to workgroups (default),
                            1 = dynamic work queue (each workgroup / wavefront claims its next tile from a
                            per-stage counter; "8 - Ecrire son megakernel", section 8.8) */
} mk_options;

/* Device pointers to canonical fp16 weights; per-layer entries are host
 * arrays of n_layers device pointers.  Borrowed only for the duration of
 * mk_load_weights (the library copies and repacks them). */
typedef struct mk_weights {
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* mlp_norm;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
} mk_weights;

/* Error record written by the device watchdog / NaN check. */
typedef struct mk_fault {
  int32_t code;  /* 0, MK_ETIMEOUT or MK_ENAN */
  int32_t cta, pc, op, step, layer, index, pad;
} mk_fault;

typedef struct mk_stats_t {
  double gpu_ms;             /* duration of the last monokernel launch (HIP events on the bound stream) */
  int32_t steps;             /* decode steps in that launch */
  int32_t pos0;              /* first position of that launch */
  int32_t grid, block, lds_bytes, ring_depth;
  int64_t stream_bytes;      /* bytes of repacked weights streamed per step (with padding) */
  int64_t weight_bytes;      /* algorithmic weight bytes per step (no padding) */
  int64_t kv_bytes_per_pos;  /* K+V bytes per cached position over all layers */
  int64_t algo_bytes;        /* algorithmic bytes of the last launch: sum over its steps */
  int32_t n_cu, occupancy;
  mk_fault fault;
  double prefill_ms;          /* last mk_prefill: GPU time of the MFMA prefill launch (0 if none ran) */
  int32_t prefill_positions;  /* positions that launch filled (the prompt's last token runs a decode step) */
  int32_t prefill_grid;       /* its workgroups (0 if none ran) */
} mk_stats_t;

typedef struct mk_ctx mk_ctx;

/* Fill *opts with the defaults (sentinel sync, 8 replicas, chosen splits, no
 * trace, 2 s watchdog, full grid).  MK_EINVAL for NULL. */
int mk_default_options(mk_options* opts);

/* Create a context on `device`, enqueueing on `hip_stream` (NULL = default
 * stream).  Sizes the one-wave launch as "8 - Ecrire son megakernel" (section
 * 8.3) prescribes -- dynamic LDS set, occupancy queried, grid = CUs x
 * occupancy -- and builds the per-workgroup instruction lists of section 8.2
 * for one decode step; allocates all device memory the library needs
 * (repacked weights, KV cache of max_seq positions, sync buffers).  *out is a
 * context owned by the library until mk_destroy.  Errors: MK_EINVAL (shape or
 * option outside the documented limits, or a device that is not gfx950),
 * MK_EOCC (the kernel does not fit a CU, or opts->grid exceeds CUs x
 * occupancy), MK_ENOMEM, MK_EHIP; text from mk_last_error(NULL). */
int mk_create(const mk_config* cfg, const mk_options* opts, int device, void* hip_stream, mk_ctx** out);

/* Copy and repack the weights (device pointers, borrowed for the call only)
 * into the per-wavefront streams the monokernel reads in order, so weights
 * flow from HBM without interruption ("7 - AMD et le monokernel", section
 * 7.5).  Resets the generation state (position 0).  Errors: MK_EINVAL (a NULL
 * pointer), MK_ENOMEM, MK_EHIP.  Synchronises. */
int mk_load_weights(mk_ctx* ctx, const mk_weights* w);

/* Prefill ("7 - AMD et le monokernel", section 7.1 names prefill among the
 * single kernel's duties): run the prompt ids[0..n) (host, each in [0,
 * vocab)) at positions 0..n-1, filling the KV cache; *t0_out = the token
 * chosen after the prompt (greedy, or drawn when sampling is on:
 * mk_set_sampling).  Positions 0..n-2 run in one persistent launch of the
 * prefill kernel: every projection as an MFMA GEMM over all positions (fp32
 * activations split into fp16 hi + lo, fp32 accumulation) and causal
 * attention tiles; the last token then runs one decode step of the
 * monokernel, which chooses t0 as every later token is chosen.  Shapes the
 * prefill kernel does not take (d_model, ffn or n_heads*head_dim not a
 * multiple of 8), and the environment variable MK_PREFILL_STEPS, run every
 * prompt token as a teacher-forced decode step instead.  Resets the
 * generation state; afterwards the position is n.  Errors: MK_ESTATE (no
 * weights loaded), MK_EINVAL (n < 1 or NULL), MK_ERANGE (n > max_seq or an id
 * outside the vocabulary), MK_ETIMEOUT, MK_ENAN, MK_EHIP.  Synchronises. */
int mk_prefill(mk_ctx* ctx, const int32_t* ids, int32_t n, int32_t* t0_out);

/* Decode ("7 - AMD et le monokernel", section 7.1: one persistent kernel,
 * no return to the host between tokens): n_steps tokens (greedy, or drawn
 * when sampling is on) in ONE launch.  Step s consumes the previous token at
 * position pos+s.  tokens_out (host, n_steps) receives the tokens;
 * logits_out (host, n_steps*vocab floats, or NULL) receives every step's
 * logits.  Errors: MK_ESTATE (before mk_prefill), MK_EINVAL (n_steps < 1),
 * MK_ERANGE (pos + n_steps > max_seq), MK_ETIMEOUT (the device watchdog
 * fired; the context then needs mk_prefill again), MK_ENAN (a NaN logit;
 * tokens are still returned), MK_EHIP.  Synchronises. */
int mk_decode(mk_ctx* ctx, int32_t n_steps, int32_t* tokens_out, float* logits_out);

/* Like mk_decode, but step s consumes tokens_in[s] (host) instead of the
 * previous token (teacher forcing).  tokens_out gets each step's choice (the
 * argmax, or the draw when sampling is on: mk_set_sampling). */
int mk_decode_forced(mk_ctx* ctx, int32_t n_steps, const int32_t* tokens_in,
                     int32_t* tokens_out, float* logits_out);

/* Generation as "7 - AMD et le monokernel" (section 7.1) describes it --
 * prefill, then decode with the kernel's own token choice: mk_prefill(ids)
 * then mk_decode(n_steps); tokens_out (host) receives n_steps + 1 tokens
 * t0..t_n.  Errors: those of the two calls. */
int mk_generate(mk_ctx* ctx, const int32_t* ids, int32_t n_prompt, int32_t n_steps, int32_t* tokens_out);

/* Token choice of every later step (prefill's t0 included): top_k = 1 (the
 * default) is greedy argmax; 2 <= top_k <= 16 draws from the top_k largest
 * logits with weights exp((z_i - z_max) / temperature), ordered by logit
 * (equal logits by increasing id), by the inverse-CDF rule: the first
 * candidate whose running weight sum exceeds u * total, else the last.  u is
 * the first 32-bit word of Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC11) with key (seed mod 2^32, seed div 2^32)
 * and counter (p, 0, 0, 0), p = the position of the token the step consumes,
 * taken as floor(word / 2^8) / 2^24.  Sampling is what "7 - AMD et le
 * monokernel" (section 7.1) names among the single kernel's duties; the
 * rule itself is the plain reading.  Weights and sums are fp32; the whole
 * choice runs inside the monokernel (every workgroup merges the per-
 * workgroup top-k lists and draws the same token).  MK_EINVAL for top_k
 * outside [1, min(16, vocab)] or, when top_k > 1, a temperature that is not
 * positive and finite; the state is then unchanged. */
int mk_set_sampling(mk_ctx* ctx, int32_t top_k, float temperature, uint64_t seed);

/* Name of the monokernel the context's last launch ran (before any launch:
 * the one a decode from the current position would run):
 * "mk_monokernel_w4h128" or, in counter sync mode, "mk_monokernel_w4h128_ctr"
 * (specialised to GEMV slices of four 512-column chunks, head_dim 128 and the
 * sync mode, used when every instruction of the schedule fits it),
 * "mk_monokernel_w4h128_long" (the sentinel-mode specialised kernel whose long
 * attention splits stream K/V through LDS by DMA, run when every split of the
 * launch's first step is longer than 32 positions) or "mk_monokernel"
 * (general).  All compute the same results; the environment variable
 * MK_GENERAL_KERNEL forces the general one.  "" for a NULL context.  The
 * string is static. */
const char* mk_kernel_name(const mk_ctx* ctx);

/* Move the generation state back to position pos (1 <= pos <= current): the
 * KV cache of positions < pos is kept and the token consumed at pos becomes
 * the next input. */
int mk_rewind(mk_ctx* ctx, int32_t pos);

/* Current position and the token the next decode step consumes. */
int mk_position(const mk_ctx* ctx, int32_t* pos, int32_t* next_token);

/* Figures of the last launch: GPU time from HIP events on the bound stream,
 * algorithmic bytes (the roofline numerator of "7 - AMD et le monokernel",
 * section 7.5: weights plus the K/V read per token), launch shape and the
 * watchdog's fault record ("8 - Ecrire son megakernel", section 8.7).  No
 * device work.  MK_EINVAL for NULL. */
int mk_stats(const mk_ctx* ctx, mk_stats_t* out);

/* Text of the context's last error (of the last failed mk_create or probe
 * for NULL).  The string belongs to the library. */
const char* mk_last_error(const mk_ctx* ctx);
/* Free every device buffer of the context (synchronises its stream first). */
void mk_destroy(mk_ctx* ctx);

/* ---- GEMV-tanh chain microbenchmark ------------------------------------
 * stages dependent stages y_i = tanh(W_i y_{i-1}) (W_i fp16 [n, n] row-major,
 * y fp32) spread over all workgroups of one persistent launch, with the same
 * streaming and synchronisation as the decoder: the per-stage cost of a
 * dependent handoff that "7 - AMD et le monokernel" (section 7.3) compares
 * between an atomic grid barrier and the NaN sentinel.  W is a device pointer
 * to [stages][n][n] fp16 (borrowed during mk_chain_create only); n a multiple
 * of 4 in [4, 16384].  Errors as for mk_create / mk_decode. */
typedef struct mk_chain mk_chain;
int mk_chain_create(int32_t n, int32_t stages, const void* W, const mk_options* opts,
                    int device, void* hip_stream, mk_chain** out);
/* x0: device [n] fp32; y: device [stages][n] fp32 (written, caller-owned).
 * One launch.  Synchronises. */
int mk_chain_run(mk_chain* ch, const float* x0, float* y);
/* Figures of the last chain run (layout of mk_stats_t). */
int mk_chain_stats(const mk_chain* ch, mk_stats_t* out);
const char* mk_chain_last_error(const mk_chain* ch);
void mk_chain_destroy(mk_chain* ch);

/* ---- host-only planning (no GPU needed) --------------------------------- */
typedef struct mk_plan_info {
  int32_t n_cta, max_ins_per_cta, n_sync_ids, lds_bytes;
  int64_t stream_chunks;     /* 1 KB chunks of repacked weights per step */
  int64_t stream_bytes, weight_bytes;
  int32_t min_wave_chunks, max_wave_chunks;
  int32_t attn_splits;
  int32_t specialised;       /* 1: the schedule runs on a specialised monokernel (see mk_kernel_name) */
} mk_plan_info;


/* Build the schedule for n_cta workgroups and check it: every consumed
 * unit has exactly one producer earlier in the step, counters match the
 * producer counts, every wave's stream is consistent.  Returns MK_OK or
 * MK_EINVAL with the reason in *msg (a static string). */
int mk_plan_check(const mk_config* cfg, const mk_options* opts, int32_t n_cta,
                  mk_plan_info* info, const char** msg);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
