// Host planner of the Muon step: validation, orientation, head blocks, owned
// runs, workspace carving, LPT-ordered tile lists and launch recipes.  Host
// code only; it makes no HIP call, so it is testable without a GPU.
#pragma once

#include <string>
#include <vector>

#include "muon.h"
#include "tables.hpp"

namespace muon {

void set_error(const std::string &msg);
const char *last_error();

struct MatrixPlan {
  muon_matrix desc;
  int32_t heads;     // >= 1
  int64_t hr;        // rows per head block
  int32_t prob0;     // first problem (global index)
  int32_t wave;
  float scale;       // fp32 shape scale sqrt(max(1, rows/cols))
  std::vector<muon_run> runs;
  bool ops32;                    // Newton-Schulz operands fp32 (else bf16)
  int64_t elem;                  // operand element bytes (4 or 2)
  int64_t ldc, ldhr;             // padded leading dims of the two copies
  int64_t orig_off[2];           // relative to the data base of the wave
  int64_t trans_off[2];          // -1 if not allocated
  int64_t u_off;                 // absolute workspace offset of the dense output
};

struct ProblemPlan {
  int32_t matrix, head;
  int32_t m, n;
  bool tall;
  double flops;
  int64_t ldm;
  int64_t mm_off[6];  // R_MA .. R_QB relative to the data base; -1 unused
  int64_t lo_off[5];  // R_MA_LO .. R_MT_LO (split-bf16 Gram chain); -1 unused
};

struct WavePlan {
  std::vector<int32_t> matrices;
  std::vector<int32_t> problems;  // global ids in LPT order (wave-local index = position)
  int64_t data_bytes = 0;
  // byte offsets of this wave's tables inside the workspace
  // tile lists per problem group and list kind (ProbGroup x TileList)
  int64_t off_prob = 0, off_k1 = 0, off_runs = 0;
  int64_t off_tiles[NGROUPS][NLISTS] = {};
  std::vector<ProbDev> probs;
  std::vector<K1Prob> k1;
  std::vector<TileDev> tiles[NGROUPS][NLISTS];
  std::vector<K3Run> runs;
  std::vector<muon_run> run_src;     // the owned run behind each K3 entry (to patch pointers)
  std::vector<int32_t> k1_matrix;    // matrix of each K1 problem
  int32_t k1_tiles = 0;
  int64_t k3_chunks = 0;
  int64_t k3_base = 0;   // index of this wave's first K3 chunk over all waves
  // persistent schedule of the large-tile groups (empty unless the options
  // ask for it): per group the queues of XCD 0..7 concatenated, their
  // bounds, the schedule as the kernel reads it, and the byte offsets of
  // these and of the group's counters in the workspace; per problem of the
  // wave the tile counts of its two lists
  std::vector<TileDev> pq[NGROUPS];
  int32_t pq_off[NGROUPS][PQ_XCDS + 1] = {};
  std::vector<PLaunch> pl[NGROUPS];
  std::vector<int32_t> pntl;
  int64_t off_pq[NGROUPS] = {}, off_pl[NGROUPS] = {}, off_pcnt[NGROUPS] = {}, off_pntl = 0;
};

// Address range of one buffer of a call, for the overlap check.
struct AddrRange {
  uintptr_t lo, hi;
  const char *what;
  int64_t index;
};

// Step of the launch schedule.
struct Launch {
  enum Kind { GEMM_OP, GEMM_F32, COPY_SCALED } kind;
  GemmRecipe r;
  bool mn;  // tile list: false = m x m (symmetric), true = m x n
};

}  // namespace muon

struct muon_plan {
  muon_options opt;
  muon_layout layout;
  std::vector<muon::MatrixPlan> mats;
  std::vector<muon::ProblemPlan> probs;
  std::vector<muon::WavePlan> waves;
  // launch schedule per problem group: [PG_F32] fp32 operands, [PG_BF16]
  // bf16 operands, [PG_BF16_BIG] bf16 large blocks (the split-bf16 Gram
  // chain; equal to [PG_BF16] for the standard form), [PG_BF16_LEAN] the
  // Gram chain with a one-product Q accumulation
  std::vector<muon::Launch> schedule[muon::NGROUPS];
  int64_t tables_bytes = 0;  // all waves' tables, at the head of the workspace
  int64_t partials_off = 0, scales_off = 0, data_off = 0, ws_bytes = 0;
  int64_t max_k1_tiles = 0, max_probs = 0;
  int64_t k0_table_bytes = 0;  // accumulation table (shares the table region)
  // update norm: per-K3-chunk sums of squares (all waves), then [norm, clip]
  int64_t nparts_off = 0, nparts_n = 0, nc_off = 0, nl1_off = 0;
  const void *norm_ws = nullptr;  // workspace of the last muon_step (its partials are current)
  std::vector<char> host_tables;  // serialized tables (pointers patched per call)
  // host buffers sized at plan creation, so a step needs no host allocation:
  // a copy of the tables to patch per call (for uploads that do not go
  // through the pinned staging), and the ranges of the overlap check
  std::vector<char> patch_host;
  std::vector<muon::AddrRange> ranges;
  // lazily created HIP resources (pinned staging, events), see abi.cpp
  void *staging[2] = {nullptr, nullptr};
  size_t staging_bytes = 0;
  void *events[2] = {nullptr, nullptr};
  bool event_live[2] = {false, false};
  int slot = 0;
  // a second stream (default priority) on which the small-block problem
  // groups run beside the large-tile ones, with the fork / join events;
  // created on the first step that has both kinds
  void *side_stream = nullptr;
  void *fork_ev = nullptr, *join_ev = nullptr;
  // phase timing (events created lazily; 4 per wave: start, K1 done, NS done, K3 done)
  bool timing = false;
  bool timed_step = false;
  int32_t timed_launches = 0;
  std::vector<void *> phase_events;
  muon_stats stats{};
};

namespace muon {
muon_status build_plan(muon_plan *p);

// The pieces of a step, shared by the entry points that run one (abi.cpp):
//  - step_check: every argument check; nothing is enqueued;
//  - step_patch: the plan's tables with this call's pointers, written to h
//    (p->host_tables.size() bytes) for a workspace at wsb;
//  - step_launch: K1, the norm, the Newton-Schulz launches and K3 on stream
//    s, reading the tables at the head of the workspace (timed: record the
//    phase events if timing is enabled; side: run the small-block groups on
//    the plan's second stream, concurrently with the large-tile groups);
//  - step_count: the plan's counters.
muon_status step_check(muon_plan *p, const void *const *grads, float *const *momenta, float *const *partitions,
                       const int32_t *skip_flag, float grad_scale, void *ws, size_t ws_bytes);
void step_patch(const muon_plan *p, char *h, const void *const *grads, float *const *momenta,
                float *const *partitions, char *wsb);
muon_status step_launch(muon_plan *p, const int32_t *skip_flag, float grad_scale, char *wsb, void *stream,
                        bool timed, bool side);
void step_count(muon_plan *p, const int32_t *skip_flag, const void *ws);
}
