// Launchers of the library's kernels (host side).
#pragma once

#include <hip/hip_runtime_api.h>

#include "tables.hpp"

namespace muon {

hipError_t launch_k0(const K0Mat *mats, int nmat, int64_t chunks, bool gbf16, int first, hipStream_t s);
// `skip` (device int32, may be NULL): kernels of a step or of the parameter
// update return at once when it holds a non-zero value.
hipError_t launch_k1(const K1Prob *probs, int nprob, int tiles, char *ws, float *partials, float beta, int nesterov,
                     float grad_scale, const int32_t *skip, bool gbf16, hipStream_t s);
hipError_t launch_kn(const K1Prob *probs, int nprob, const float *partials, float *scales, float eps,
                     const int32_t *skip, hipStream_t s);
// nparts (may be NULL): per-chunk sums of squares of the written values,
// chunk i of this launch at nparts[pbase + i]
hipError_t launch_k3(const K3Run *runs, int nrun, int64_t chunks, const int32_t *skip, float *nparts, int64_t pbase,
                     hipStream_t s);
hipError_t launch_kc(const ProbDev *probs, const K1Prob *k1, int nprob, char *ws, const float *scales,
                     const int32_t *skip, hipStream_t s);
// flag = 1 if any element of the matrices is not finite, else 0
hipError_t launch_finite(const K0Mat *mats, int nmat, int64_t chunks, bool gbf16, int32_t *flag, hipStream_t s);
// norm = sqrt(sum of nparts[0..n)) (fp64, fixed order, through l1: one
// double per 8192 partials); nc[0] = norm, nc[1] = clip factor; copied to
// user_out[0..2) when that is not NULL
hipError_t launch_norm_clip(const float *nparts, int64_t n, double *l1, float max_norm, float *nc, float *user_out,
                            const int32_t *skip, hipStream_t s);
constexpr int64_t kNormSpan = 8192;  // partials per level-1 sum
// param = param * (1 - lr wd) - (lr clip) upd on every run
hipError_t launch_apply(const KARun *runs, int nrun, int64_t chunks, const float *nc, float lr, float wd,
                        const int32_t *skip, hipStream_t s);

// One grouped Newton-Schulz GEMM launch over a tile list.
struct GemmArgs {
  const ProbDev *probs;
  const TileDev *tiles;
  char *ws;
  const float *scales;
  GemmRecipe r;
  const int32_t *skip;   // may be NULL; non-zero: the launch does nothing
};
hipError_t launch_gemm(bool bf16_operands, const GemmArgs &a, int ntiles, hipStream_t s);

// The fused Newton-Schulz of the PG_HEAD blocks: one workgroup per entry of
// the tile list (its tm, tn are 0) runs the block's whole iteration.
struct HeadArgs {
  const ProbDev *probs;
  const TileDev *tiles;
  char *ws;
  const float *scales;
  const int32_t *skip;   // may be NULL; non-zero: the launch does nothing
  float a, b, c;
  int32_t steps;         // >= 1
  int32_t standard;      // 1: standard form, 0: Gram form
};
hipError_t launch_head(const HeadArgs &a, int nprob, hipStream_t s);
hipError_t launch_gemm256(const GemmArgs &a, int ntiles, hipStream_t s);

// The persistent launch of a large-tile group: one workgroup per CU (8 XCDs
// of 32), each walking the queue of its XCD.
struct PersistArgs {
  const ProbDev *probs;
  char *ws;
  const float *scales;
  const int32_t *skip;         // may be NULL; non-zero: the launch does nothing
  const PLaunch *launches;     // the group's schedule
  const TileDev *items;        // the queues of XCD 0 .. 7, concatenated
  const int32_t *ntl;          // [problem][2]: tiles of its m x m and m x n lists
  int32_t *counters;           // PQ_PAD-strided dequeue and completion counters, zero
  int32_t qoff[PQ_XCDS + 1];   // queue x = items[qoff[x], qoff[x + 1])
};
hipError_t launch_persist(const PersistArgs &a, bool split, hipStream_t s);

}  // namespace muon
