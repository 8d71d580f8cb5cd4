// mk_plan.cpp -- builds and checks the static schedule of the monokernel.
//
// The structure follows the interpreter of "8 - Ecrire son megakernel"
// (section 8.2): every workgroup owns an instruction list; an instruction
// names its input dependency and the output it produces.  Here the lists are
// built once per context for one decode step (the device repeats them for
// every step), and each wavefront also gets the exact sequence of 1 KB weight
// chunks it will stream, so that weights flow continuously from HBM
// ("7 - AMD et le monokernel", section 7.5).  check_plan is the static
// validator run before any launch ("8 - Ecrire son megakernel", section 8.7,
// static verification): each unit has one producer, counter targets match the
// producer counts, streams match the instructions.
#include "mk_plan.h"

#include <algorithm>

namespace mk {

// rings | staged vector | scratch | residual rows | small fields (flags,
// wave sums, argmax keys, trace scratch, barrier, ring tags and counts).
int lds_bytes_for(int kpad_max) {
  return kWaves * kRing * 1024 + kpad_max * 4 + kScratchFloats * 4 + kResidRows * 4 + kSmallBytes;
}

int choose_splits(int n_cta, int nkv, int max_seq) {
  int s = n_cta / std::max(1, nkv);
  s = std::min(s, 64);
  s = std::min(s, std::max(1, (max_seq + 7) / 8));
  return std::max(1, s);
}

int Plan::mat_cols(int mat) const {
  if (dm.chain) return dm.chain_n;
  if (mat == 7 * dm.L) return dm.d;
  switch (mat % 7) {
    case MO: return dm.nq * dm.hd;
    case MD: return dm.f;
    default: return dm.d;
  }
}

int Plan::mat_rows(int mat) const {
  if (dm.chain) return dm.chain_n;
  if (mat == 7 * dm.L) return dm.V;
  switch (mat % 7) {
    case MQ: return dm.nq * dm.hd;
    case MK: case MV: return dm.nkv * dm.hd;
    case MO: case MD: return dm.d;
    default: return dm.f;
  }
}

namespace {

// Stage ids within one step (the attention stage also merges its splits).
int sid_qkv(int l) { return 5 * l + 0; }
int sid_att(int l) { return 5 * l + 1; }
int sid_o(int l) { return 5 * l + 2; }
int sid_up(int l) { return 5 * l + 3; }
int sid_dn(int l) { return 5 * l + 4; }

// Units of a stage dealt to workgroups: contiguous balanced ranges when there
// are at least as many units as workgroups, else one unit for each of the
// first U workgroups (consecutive workgroups sit on different XCDs).
void split_units(int U, int n, int c, int* u0, int* nu) {
  if (U >= n) {
    int64_t a = (int64_t)U * c / n, b = (int64_t)U * (c + 1) / n;
    *u0 = (int)a;
    *nu = (int)(b - a);
  } else {
    *u0 = c;
    *nu = c < U ? 1 : 0;
  }
}

struct Stage {
  uint8_t op;
  int layer, U, upr, K, sync_in, sync_out;
};

// Matrix and row of GEMV row r (0..upr-1) of global unit g.
void row_source(const Plan& p, const Stage& st, int g, int r, int* mat, int* row) {
  const Dims& dm = p.dm;
  const int l = st.layer;
  switch (st.op) {
    case OP_QKV: {
      const int hh = dm.hd / 2;
      int kind, head, i;
      if (g < dm.nq * hh) { kind = MQ; head = g / hh; i = g % hh; }
      else if (g < (dm.nq + dm.nkv) * hh) { kind = MK; g -= dm.nq * hh; head = g / hh; i = g % hh; }
      else { kind = MV; g -= (dm.nq + dm.nkv) * hh; head = g / hh; i = g % hh; }
      *mat = 7 * l + kind;
      *row = head * dm.hd + i + r * hh;
      return;
    }
    case OP_UPGATE: *mat = 7 * l + (r == 0 ? MG : MU); *row = g; return;
    case OP_OPROJ: *mat = 7 * l + MO; *row = g; return;
    case OP_DOWN: *mat = 7 * l + MD; *row = g; return;
    case OP_LMHEAD: *mat = 7 * dm.L; *row = g; return;
    case OP_CHAIN: *mat = l; *row = g; return;
    default: *mat = -1; *row = -1; return;
  }
}

// K split for nu units of upr rows with kc_raw chunks per row: the power of
// two ks (dividing the wavefront count) that minimises the busiest
// wavefront's chunk count, with at most 4 chunks per slice (the activation
// slice lives in registers).  Rows are zero-padded to a multiple of ks chunks.
// ks = 0 when no split fits (rows too long for the registers and too many
// rows for the merge scratch).
void choose_split(int nu, int upr, int kc_raw, int* ks_out, int* cps_out) {
  int best = -1, best_ks = 0, best_cps = 1;
  for (int ks = 1; ks <= kWaves; ks *= 2) {
    const int kc = (kc_raw + ks - 1) / ks * ks, cps = kc / ks;
    if (cps > 4) continue;
    if (ks > 1 && (int64_t)nu * upr * ks > kScratchFloats) continue;
    const int rg = kWaves / ks;
    // busiest wavefront: its chunks plus one chunk-equivalent per row for the
    // wavefront reduction, plus the cross-wavefront merge when K is split
    const int load = ((nu + rg - 1) / rg) * upr * (cps + 1) + (ks > 1 ? 2 : 0);
    if (best < 0 || load < best) {
      best = load;
      best_ks = ks;
      best_cps = cps;
    }
  }
  *ks_out = best_ks;
  *cps_out = best_cps;
}

bool is_gemv(uint8_t op) {
  return op == OP_QKV || op == OP_OPROJ || op == OP_UPGATE || op == OP_DOWN || op == OP_LMHEAD || op == OP_CHAIN;
}

}  // namespace

int plan_lds_bytes(const Dims& dm) {
  auto kpad = [](int K) { return ((K + kChunkHalfs - 1) / kChunkHalfs + 7) / 8 * 8 * kChunkHalfs; };
  if (dm.chain) return lds_bytes_for(kpad(dm.chain_n));
  const int G = dm.nkv > 0 ? dm.nq / dm.nkv : 1;
  return lds_bytes_for(std::max({kpad(dm.d), kpad(dm.nq * dm.hd), kpad(dm.f), att_stage_floats(G, dm.hd)}));
}

std::string build_plan(const Dims& dm, int n_cta, int S, int R, int sync_mode, Plan* out) {
  Plan& p = *out;
  p = Plan();
  p.dm = dm;
  p.n_cta = n_cta;
  p.R = R;
  p.sync_mode = sync_mode;
  if (n_cta < 1) return "grid must have at least one workgroup";
  if (!(R == 1 || R == 2 || R == 4 || R == 8)) return "xcd_replicas must be 1, 2, 4 or 8";

  std::vector<Stage> stages;
  int kpad_max = 0;
  // staged row length upper bound: rows padded to a multiple of 8 chunks at most
  auto kpad = [](int K) { return ((K + kChunkHalfs - 1) / kChunkHalfs + 7) / 8 * 8 * kChunkHalfs; };
  if (dm.chain) {
    if (dm.chain_n < 4 || dm.chain_n % 4 || dm.chain_n > kMaxK) return "chain n must be a multiple of 4 in [4, 16384]";
    if (dm.chain_stages < 1) return "chain needs at least one stage";
    for (int i = 0; i < dm.chain_stages; ++i)
      stages.push_back({OP_CHAIN, i, dm.chain_n, 1, dm.chain_n, i == 0 ? -1 : i - 1, i});
    p.n_sync = dm.chain_stages;
    p.S = 1;
    kpad_max = kpad(dm.chain_n);
    p.weight_bytes = (int64_t)dm.chain_stages * dm.chain_n * dm.chain_n * 2;
  } else {
    const int qd = dm.nq * dm.hd;
    if (dm.L < 1 || dm.d < 4 || dm.nq < 1 || dm.nkv < 1 || dm.f < 4 || dm.V < 2 || dm.max_seq < 2)
      return "dimensions must be positive (d, ffn >= 4, vocab >= 2, max_seq >= 2)";
    if (dm.nq % dm.nkv) return "n_heads must be a multiple of n_kv_heads";
    if (!(dm.hd == 64 || dm.hd == 128 || dm.hd == 256)) return "head_dim must be 64, 128 or 256";
    if (dm.d % 4 || dm.f % 4) return "d_model and ffn must be multiples of 4";
    if (dm.d > kMaxK || dm.f > kMaxK || qd > kMaxK) return "d_model, ffn and n_heads*head_dim must be at most 16384";
    const int G = dm.nq / dm.nkv;
    // attention combines at most 8 / (hd / 64) query heads per pass through the scratch
    if (kWaves * std::min(G, 8 / (dm.hd / 64)) * (dm.hd + 2) > kScratchFloats)
      return "attention combine does not fit the LDS scratch";
    p.S = S > 0 ? S : choose_splits(n_cta, dm.nkv, dm.max_seq);
    if (p.S < 1 || p.S > 64) return "attn_splits must be in [1, 64]";
    const int hh = dm.hd / 2;
    for (int l = 0; l < dm.L; ++l) {
      stages.push_back({OP_QKV, l, (dm.nq + 2 * dm.nkv) * hh, 2, dm.d, l == 0 ? -1 : sid_dn(l - 1), sid_qkv(l)});
      stages.push_back({OP_ATT, l, dm.nkv * p.S, 0, 0, sid_qkv(l), sid_att(l)});
      stages.push_back({OP_OPROJ, l, dm.d, 1, qd, sid_att(l), sid_o(l)});
      stages.push_back({OP_UPGATE, l, dm.f, 2, dm.d, sid_o(l), sid_up(l)});
      stages.push_back({OP_DOWN, l, dm.d, 1, dm.f, sid_up(l), sid_dn(l)});
    }
    stages.push_back({OP_LMHEAD, dm.L, dm.V, 1, dm.d, sid_dn(dm.L - 1), 5 * dm.L});
    stages.push_back({OP_ARGMAX, dm.L, 1, 0, 0, 5 * dm.L, -1});
    p.n_sync = 5 * dm.L + 1;
    kpad_max = std::max({kpad(dm.d), kpad(qd), kpad(dm.f), att_stage_floats(G, dm.hd)});
    const int64_t per_layer = (int64_t)(qd + 2 * dm.nkv * dm.hd) * dm.d + (int64_t)dm.d * qd + 3LL * dm.f * dm.d;
    p.weight_bytes = 2 * (per_layer * dm.L + (int64_t)dm.V * dm.d + (int64_t)dm.d * (2 * dm.L + 1) + dm.d);
  }
  p.lds_bytes = lds_bytes_for(kpad_max);
  if (p.lds_bytes != plan_lds_bytes(dm)) return "internal: LDS footprint mismatch";
  if (p.lds_bytes > 160 * 1024) return "the LDS footprint exceeds 160 KB (row length too large for the ring)";

  // producer counts
  p.n_prod.assign(p.n_sync, 0);
  int lm_count = 0;
  for (const Stage& st : stages) {
    if (st.op == OP_ARGMAX) continue;
    for (int c = 0; c < n_cta; ++c) {
      int u0, nu;
      split_units(st.U, n_cta, c, &u0, &nu);
      // every workgroup publishes an argmax key (possibly empty): the keys
      // double as the end-of-step signal of every workgroup
      if (nu > 0 || st.op == OP_LMHEAD) {
        p.n_prod[st.sync_out]++;
        if (st.op == OP_LMHEAD) lm_count++;
      }
    }
  }
  p.lm_slots = lm_count;

  // instruction lists
  p.ins_off.assign(n_cta + 1, 0);
  for (int c = 0; c < n_cta; ++c) {
    p.ins_off[c] = (int)p.ins.size();
    for (const Stage& st : stages) {
      Ins in{};
      in.op = st.op;
      in.layer = (int16_t)st.layer;
      in.sync_in = (int16_t)st.sync_in;
      in.sync_out = (int16_t)st.sync_out;
      in.n_in = (int16_t)(st.sync_in >= 0 ? p.n_prod[st.sync_in] : 0);
      in.slot = -1;
      if (st.op == OP_ARGMAX) {
        in.u0 = 0;
        in.nu = p.lm_slots;
        p.ins.push_back(in);
        continue;
      }
      int u0, nu;
      split_units(st.U, n_cta, c, &u0, &nu);
      if (nu == 0 && st.op != OP_LMHEAD) continue;
      in.u0 = u0;
      in.nu = nu;
      if (is_gemv(st.op)) {
        int ks, cps;
        choose_split(std::max(nu, 1), st.upr, (st.K + kChunkHalfs - 1) / kChunkHalfs, &ks, &cps);
        if (ks == 0) return "no K split fits: too many GEMV rows per workgroup for this row length (use a larger grid)";
        in.upr = (uint8_t)st.upr;
        in.ks = (uint8_t)ks;
        in.cps = (uint8_t)cps;
        in.kpad = ks * cps * kChunkHalfs;
      }
      if (st.op == OP_LMHEAD) in.slot = c;
      p.ins.push_back(in);
    }
    p.max_ins = std::max(p.max_ins, (int)p.ins.size() - p.ins_off[c]);
  }
  p.ins_off[n_cta] = (int)p.ins.size();

  // wave streams
  p.wave_off.assign((size_t)n_cta * kWaves, 0);
  p.wave_n.assign((size_t)n_cta * kWaves, 0);
  for (int c = 0; c < n_cta; ++c) {
    for (int w = 0; w < kWaves; ++w) {
      p.wave_off[c * kWaves + w] = (int64_t)p.chunks.size();
      for (int k = p.ins_off[c]; k < p.ins_off[c + 1]; ++k) {
        const Ins& in = p.ins[k];
        if (!is_gemv(in.op)) continue;
        const int ks = in.ks, rg = kWaves / ks, ki = w % ks, gi = w / ks;
        Stage st{in.op, in.layer, 0, in.upr, 0, 0, 0};
        for (int u = gi; u < in.nu; u += rg)
          for (int r = 0; r < in.upr; ++r) {
            int mat, row;
            row_source(p, st, in.u0 + u, r, &mat, &row);
            for (int cc = 0; cc < in.cps; ++cc) p.chunks.push_back({mat, row, ki * in.cps + cc});
          }
      }
      p.wave_n[c * kWaves + w] = (int32_t)((int64_t)p.chunks.size() - p.wave_off[c * kWaves + w]);
    }
  }
  return check_plan(p);
}

std::string check_plan(const Plan& p) {
  const Dims& dm = p.dm;
  if ((int)p.ins_off.size() != p.n_cta + 1) return "instruction offsets have the wrong length";
  // every unit of every (op, layer) produced exactly once; stage order is monotone
  std::vector<std::vector<int>> cover;   // indexed by sync id
  cover.resize(p.n_sync);
  std::vector<int> prod(p.n_sync, 0);
  for (int c = 0; c < p.n_cta; ++c) {
    int last = -1;
    bool has_argmax = false;
    for (int k = p.ins_off[c]; k < p.ins_off[c + 1]; ++k) {
      const Ins& in = p.ins[k];
      if (in.op == OP_ARGMAX) {
        if (in.n_in != p.lm_slots || in.sync_in != p.n_sync - 1) return "argmax must wait for every LM-head slot";
        if (k != p.ins_off[c + 1] - 1) return "argmax must close the step";
        has_argmax = true;
        continue;
      }
      if (in.sync_out < 0 || in.sync_out >= p.n_sync) return "sync id out of range";
      if (in.sync_out <= last) return "instructions out of stage order";
      last = in.sync_out;
      if (in.sync_in >= in.sync_out) return "an instruction waits for a later stage";
      if (in.sync_in >= 0 && in.n_in != p.n_prod[in.sync_in]) return "counter target differs from the producer count";
      if (in.nu < 0 || (in.nu == 0 && in.op != OP_LMHEAD)) return "empty instruction";
      prod[in.sync_out]++;
      std::vector<int>& cv = cover[in.sync_out];
      if ((int64_t)in.u0 + in.nu > (int64_t)1 << 30) return "unit range overflow";
      if ((int)cv.size() < in.u0 + in.nu) cv.resize(in.u0 + in.nu, 0);
      for (int u = in.u0; u < in.u0 + in.nu; ++u) cv[u]++;
      if (in.upr) {
        if (kWaves % in.ks) return "K slices must divide the wavefront count";
        if (in.cps < 1 || in.cps > 4) return "chunks per slice must be in [1, 4]";
        if (in.kpad > kMaxK) return "row too long";
        if (in.ks > 1 && in.nu * in.upr * in.ks > kScratchFloats) return "K-slice partials do not fit the LDS scratch";
        if ((in.op == OP_OPROJ || in.op == OP_DOWN) && in.nu > kResidRows) return "residual rows do not fit the LDS";
      }
      if (in.op == OP_LMHEAD && (in.slot < 0 || in.slot >= p.lm_slots)) return "bad argmax slot";
    }
    if (!dm.chain && !has_argmax) return "a workgroup never reads the argmax";
  }
  for (int s = 0; s < p.n_sync; ++s) {
    if (prod[s] != p.n_prod[s]) return "producer count mismatch";
    if (prod[s] == 0) return "a stage has no producer";
    for (int v : cover[s])
      if (v != 1) return "a unit is produced zero or several times";
  }
  // stage sizes
  if (!dm.chain) {
    const int hh = dm.hd / 2;
    for (int l = 0; l < dm.L; ++l) {
      if ((int)cover[sid_qkv(l)].size() != (dm.nq + 2 * dm.nkv) * hh) return "QKV units incomplete";
      if ((int)cover[sid_att(l)].size() != dm.nkv * p.S) return "attention units incomplete";
      if ((int)cover[sid_o(l)].size() != dm.d || (int)cover[sid_dn(l)].size() != dm.d) return "residual rows incomplete";
      if ((int)cover[sid_up(l)].size() != dm.f) return "MLP units incomplete";
    }
    if ((int)cover[5 * dm.L].size() != dm.V) return "LM-head rows incomplete";
  } else {
    for (int i = 0; i < dm.chain_stages; ++i)
      if ((int)cover[i].size() != dm.chain_n) return "chain rows incomplete";
  }
  // wave streams match the instruction lists
  int64_t total = 0;
  for (int c = 0; c < p.n_cta; ++c)
    for (int w = 0; w < kWaves; ++w) {
      int64_t n = 0;
      for (int k = p.ins_off[c]; k < p.ins_off[c + 1]; ++k) {
        const Ins& in = p.ins[k];
        if (!in.upr) continue;
        const int rg = kWaves / in.ks;
        n += (int64_t)units_of_group(in.nu, rg, w / in.ks) * in.upr * in.cps;
      }
      if (n != p.wave_n[c * kWaves + w]) return "wave stream length differs from its instructions";
      if (p.wave_off[c * kWaves + w] != total) return "wave streams are not contiguous";
      total += n;
    }
  if (total != (int64_t)p.chunks.size()) return "stream size mismatch";
  for (const ChunkSrc& s : p.chunks) {
    if (s.row < 0 || s.row >= p.mat_rows(s.mat)) return "chunk row out of range";
    if (s.cc < 0 || s.cc >= (p.mat_cols(s.mat) + kChunkHalfs - 1) / kChunkHalfs + 7) return "chunk column out of range";
  }
  return "";
}

}  // namespace mk
