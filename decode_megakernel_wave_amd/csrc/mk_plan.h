// mk_plan.h -- host-side schedule: per-workgroup instruction lists, the
// per-wavefront weight streams, and the static checks run before a launch.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "mk_layout.h"

namespace mk {

struct Dims {
  int L = 0, d = 0, nq = 0, nkv = 0, hd = 0, f = 0, V = 0, max_seq = 0;
  bool chain = false;
  int chain_n = 0, chain_stages = 0;
};

// Source of one 1 KB chunk of a wavefront's stream: matrix, row, 512-column chunk.
struct ChunkSrc {
  int32_t mat, row, cc;
};

// Matrix ids: decoder layer l uses 7*l + {0:q,1:k,2:v,3:o,4:gate,5:up,6:down};
// the LM head is 7*L; chain stage i is matrix i.
enum MatKind { MQ = 0, MK = 1, MV = 2, MO = 3, MG = 4, MU = 5, MD = 6 };

struct Plan {
  Dims dm;
  int n_cta = 0, S = 1, R = 1, sync_mode = 0;
  int n_sync = 0, lm_slots = 0, max_ins = 0, lds_bytes = 0;
  std::vector<Ins> ins;              // all lists, concatenated
  std::vector<int32_t> ins_off;      // [n_cta + 1]
  std::vector<int32_t> n_prod;       // producers per sync id
  std::vector<int64_t> wave_off;     // [n_cta * kWaves] (chunks)
  std::vector<int32_t> wave_n;       // [n_cta * kWaves]
  std::vector<ChunkSrc> chunks;      // concatenated wave streams
  int64_t weight_bytes = 0;          // algorithmic weight bytes per step
  int64_t stream_bytes() const { return (int64_t)chunks.size() * kChunkHalfs * 2; }
  // row length (columns) of a matrix id
  int mat_cols(int mat) const;
  int mat_rows(int mat) const;
};

// Returns "" on success or a reason.  S = attention splits (0 = choose).
std::string build_plan(const Dims& dm, int n_cta, int S, int R, int sync_mode, Plan* out);
std::string check_plan(const Plan& p);
int lds_bytes_for(int kpad_max);
int plan_lds_bytes(const Dims& dm);  // LDS footprint of the monokernel for these dims (any grid)
int choose_splits(int n_cta, int nkv, int max_seq);

}  // namespace mk
