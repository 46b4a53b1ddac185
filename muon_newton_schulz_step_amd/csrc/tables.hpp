// Tables the host planner builds and the kernels read, plus the compile-time
// tile shapes both sides agree on.  Plain structs, identical on host and
// device; the host uploads them into the head of the workspace once per call.
#pragma once

#include <stdint.h>

namespace muon {

// Buffers a Newton-Schulz problem owns in the workspace ("roles").  The
// per-launch recipe names roles; the problem table maps them to offsets.
enum Role : int {
  R_XR0 = 0,  // X, wide orientation (m x n), parity 0   [operand dtype]
  R_XC0,      // X^T (n x m), parity 0                  [operand dtype]
  R_XR1,      // X, parity 1
  R_XC1,      // X^T, parity 1
  R_MA,       // standard: A = X X^T ;  gram: R         [op dtype / fp32]
  R_MB,       // standard: C = aI + bA + cA^2 ;  gram: P [op dtype / fp32]
  R_Q0,       // gram: Q, parity 0                      [fp32]
  R_Q1,       // gram: Q, parity 1                      [fp32]
  R_MT,       // gram: P R                              [fp32]
  R_QB,       // gram: Q in the operand dtype           [operand dtype]
  R_U,        // unscaled output, original orientation, dense per matrix
  // split-bf16 Gram chain (large blocks): the low halves of R, P, Q0, Q1, T;
  // the high halves live in R_MA, R_MB, R_Q0, R_Q1, R_MT as bf16
  R_MA_LO, R_MB_LO, R_Q0_LO, R_Q1_LO, R_MT_LO,
  NROLES
};

// Output tile edges of the grouped GEMMs (square tiles; symmetric outputs
// list only tm <= tn).  bf16 problems whose small side reaches BIG_TILE use
// the large-tile kernel.
constexpr int GEMM_TILE = 128;
constexpr int BIG_TILE = 256;
#ifndef MUON_BIG_TILE_MIN_M
#define MUON_BIG_TILE_MIN_M 256
#endif
constexpr int BIG_TILE_MIN_M = MUON_BIG_TILE_MIN_M;

// Problem groups of a wave: fp32 operands; bf16 with m < BIG_TILE; bf16
// blocks fused into one workgroup each (below); bf16 with m >= BIG_TILE;
// and, in the Gram form only, bf16 blocks with
// m >= GRAM_LEAN_MIN_M, whose chain accumulates Q with one bf16 product
// (below).  Tile lists per group: m x m and m x n, at each tile size.
enum ProbGroup : int { PG_F32 = 0, PG_BF16 = 1, PG_HEAD = 2, PG_BF16_BIG = 3, PG_BF16_LEAN = 4, NGROUPS };

// bf16 blocks with m <= this (at least BF16_MIN_M, below), either form, at
// least one step: the whole iteration of a block runs in one workgroup
// (PG_HEAD; its tile list holds one entry per block, and the group has no
// launch schedule).
constexpr int HEAD_MAX_M = 128;

// Gram form, bf16 blocks with m >= this: Q <- P Q is one bf16 product of
// the high halves, stored as bf16 (three-segment split products for the
// R chain and the square of R, as for smaller blocks).  Emulated error on
// Gaussian inputs: 1.2e-2 at 2048 x 2048, 1.4e-2 at 1024 x 1024 (the full
// split chain: 6.9e-3, 8.8e-3), falling with the block size.
constexpr int GRAM_LEAN_MIN_M = 2048;
enum TileList : int { TL_MM128 = 0, TL_MN128, TL_MM256, TL_MN256, NLISTS };

// Newton-Schulz blocks whose small side is below this run on fp32 operands
// even when bf16 is asked for: with few rows, the bf16 rounding of the m x m
// polynomial matrix dominates the error and is not averaged out.
constexpr int BF16_MIN_M = 64;

// One Newton-Schulz problem (a matrix or one head block).
struct ProbDev {
  int32_t m, n;          // wide orientation, m <= n
  int32_t matrix;        // index of the source matrix
  int32_t flags;         // PF_* bits
  int64_t off[NROLES];   // byte offsets of the role buffers in the workspace
  int32_t ld[NROLES];    // leading dimension of each role buffer (elements)
  int32_t pad_[1];
};
constexpr int32_t PF_TALL = 1;  // block has more rows than columns: U is stored transposed

// One K1 problem: where a block of a matrix comes from and where its two
// copies (original layout and transposed) go.
struct K1Prob {
  const void *grad;      // matrix base (per call)
  float *mom;            // matrix base (per call)
  int64_t row0;          // first row of the block in the matrix
  int64_t cols;          // matrix columns = block columns
  int64_t orig_off;      // ws byte offset of the original-layout copy
  int64_t trans_off;     // ws byte offset of the transposed copy
  int32_t hr;            // block rows
  int32_t orig_ld, trans_ld;
  int32_t tile0;         // first K1 tile of this problem (prefix over the wave)
  int32_t tiles_c;       // tiles along the columns
  int32_t ntiles;
  int32_t xbf16;         // 1: the copies are bf16, 0: fp32
  int32_t pad_;
};
constexpr int K1_TILE = 64;  // K1 tiles are 64 x 64 elements

// One owned run of the writeback.
struct K3Run {
  const void *src;       // dense rows x cols update of the matrix (original orientation)
  float *dst;            // partition base + local offset of the run
  int64_t first;         // first element of the run in the flattened matrix
  int64_t length;
  int64_t chunk0;        // first K3 chunk of this run (prefix)
  float scale;           // fp32 shape scale
  int32_t src_bf16;      // 1: src is bf16, 0: fp32
};
constexpr int K3_CHUNK = 4096;  // elements per K3 workgroup

// One owned run of the parameter update (the same runs as the writeback).
struct KARun {
  float *param;          // fp32 master partition base + local offset of the run
  const float *upd;      // update partition base + the same offset
  int64_t length;
  int64_t chunk0;        // first chunk of this run (prefix)
};
constexpr int KA_CHUNK = 4096;

// One matrix of an accumulation call.
struct K0Mat {
  float *acc;
  const void *g;
  int64_t numel;
  int64_t chunk0;
};
constexpr int K0_CHUNK = 4096;

// GEMM tile list entry.
struct TileDev {
  int32_t prob;
  int16_t tm, tn;
};

// Recipe of one grouped GEMM launch: C = scale^p (cd D + cacc A B^T) + cdiag I,
// stored to up to two roles.  Operands are row-major with K contiguous.
struct GemmRecipe {
  int8_t rA, rB, rD, rS0, rS1;  // roles; -1 = none
  int8_t dimM, dimN, dimK;      // 0 -> m, 1 -> n
  int32_t flags;                // GF_* bits
  float cd, cacc, cdiag;
  int32_t scale_pow;            // 0, 1 or 2: power of the per-problem norm scale
  // Extra K segments summed into the same accumulators (split products):
  // segment s >= 1 multiplies roles (rA2[s-1], rB2[s-1]) over the same K.
  int8_t nseg;                  // 1 or 3
  int8_t rA2[2], rB2[2];
  int8_t rD2;                   // low half of D when GF_D_SPLIT
  int8_t pad_[2];
};
constexpr int32_t GF_SYM = 1;        // output symmetric; tiles list tm <= tn, mirror written
constexpr int32_t GF_D_F32 = 2;      // D is fp32 (else operand dtype)
constexpr int32_t GF_S0_F32 = 4;     // S0 stored fp32
constexpr int32_t GF_S1_F32 = 8;     // S1 stored fp32
constexpr int32_t GF_S0_TRANS = 16;  // S0 stored transposed
constexpr int32_t GF_S1_TRANS = 32;  // S1 stored transposed
constexpr int32_t GF_S0_PROBT = 64;  // S0 transposed iff the problem has PF_TALL
constexpr int32_t GF_DIAG = 128;     // add cdiag on the diagonal
constexpr int32_t GF_SPLIT_OUT = 256;  // S0 = bf16(v), S1 = bf16(v - S0): a hi/lo pair
constexpr int32_t GF_D_SPLIT = 512;    // D = bf16 hi (rD) + bf16 lo (rD2)

// Persistent schedule of a large-tile group (one launch for every product of
// every problem): a queue of work items per XCD.  An item is a TileDev whose
// prob field holds the problem (wave-local index) in its low 24 bits and the
// launch of the group's schedule in its high 8 bits.
constexpr int PQ_XCDS = 8;
constexpr int32_t PQ_PROB_MASK = 0xFFFFFF;
constexpr int PQ_LAUNCH_SHIFT = 24;
constexpr int PQ_MAX_LAUNCHES = 255;
// Counters, one per 128-byte line so that no two XCDs ever touch one line:
// counters[PQ_PAD x] is XCD x's dequeue position, counters[PQ_PAD (PQ_XCDS + p)]
// the finished tiles of problem p.  Zero when the launch starts.
constexpr int PQ_PAD = 32;

// One launch of the schedule as the persistent kernel reads it: the recipe
// and how many launches over each tile list precede it, so that product k
// of problem p may start once p has finished
//   mm_before * (tiles of its m x m list) + mn_before * (tiles of its m x n list).
struct PLaunch {
  GemmRecipe r;
  int32_t mm_before, mn_before;
};

}  // namespace muon
