// Fused Newton-Schulz for blocks whose small side m is at most 128 (the
// 128-row head blocks of a per-head split, and small matrices), bf16 operands
// on the m x n side.  One 256-thread workgroup runs a block's whole iteration,
// so the m x m matrices never leave the CU and a block costs one launch slot
// instead of one tile in each of the schedule's launches.
//
// Gram form (the iteration on the small side's Gram matrix: R = X0 X0^T,
// P = a I + b R + c R^2, Q <- P Q, R <- P R P, output Q X0):
//   1. stream X0 (m x n, rows K-contiguous) through LDS, R = s^2 X0 X0^T in
//      fp32 accumulators (bf16 MFMA), kept in LDS as fp32;
//   2. the T chain steps on fp32 MFMA with R and P in LDS and Q in registers;
//   3. stream X0^T (n x m) through LDS, Y^T = s X0^T (Q_hi + Q_lo) with Q as
//      a bf16 pair (hi = bf16(Q), lo = bf16(Q - hi); two bf16 MFMAs into one
//      fp32 accumulator), and store Y in the block's output orientation.
// R, P and Q are fp32 as on the tiled path for these blocks.  The output
// product takes Q to about 16 significant bits instead of bf16's 8: where
// the block is square or nearly so, Q spans a wide range and its bf16
// rounding alone puts the output 1.4e-2 to 2e-2 from the exact iteration on
// Gaussian inputs, the pair about 4e-3.  The second product costs no time:
// this phase is bound by streaming X0^T.
//
// Register-resident operands.  Every chain matrix is a polynomial in R, so
// all of them are symmetric and commute.  Wave w owns column block w
// (columns 32w .. 32w+31) of the matrices it computes; an MFMA accumulator
// tile holds column j = 32w + lane % 32 and rows 8 (r / 4) + 4 (lane / 32) +
// (r % 4) in register r, which is exactly the B-operand layout of the fp32
// 32x32x2 MFMA for the K pairs (8 q + e, 8 q + 4 + e).  So P Q and P T are
// formed as P times the wave's own column block (A operand from LDS, B from
// registers), and R P as R times the column block of P.  The matrices kept in
// LDS are written exactly symmetric (each off-diagonal pair from one computed
// value), so an LDS operand read along a row equals the read along a column.
#include <hip/hip_runtime.h>

#include "elem.hpp"
#include "tables.hpp"

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int HM = HEAD_MAX_M;        // 128: rows of every on-chip matrix
constexpr int NTHR = 256;             // 4 waves
constexpr int KC = 128;               // staged row length (bf16): the m side, or 128 columns of n
constexpr int SROW = KC + 8;          // bf16 per staged row: 272 bytes
constexpr int SBUF = HM * SROW * 2;   // 34816 bytes: 128 staged rows
constexpr int FROW = HM + 4;          // floats per row of an fp32 matrix: 528 bytes
constexpr int FMAT = HM * FROW * 4;   // 67584 bytes
constexpr int YC = 64;                // rows of X0^T per output chunk
constexpr int OROW = YC + 8;          // bf16 per row of the staged output (wide blocks): 144 bytes
// phase 1: two staging buffers of 128 rows; phase 2: R and P; phase 3: Q_hi,
// Q_lo, two staging buffers of 64 rows, the staged output
constexpr int Y_IN = 2 * SBUF, Y_OUT = 2 * SBUF + SBUF;
constexpr int OBUF = HM * OROW * 2;   // 18432 >= YC * SROW * 2 (tall blocks)
constexpr int LDS_BYTES = 2 * FMAT;   // 135168
static_assert(Y_OUT + OBUF <= LDS_BYTES && YC * SROW * 2 <= OBUF, "phase 3 fits the pool");
static_assert(HM == 128 && KC == 128 && YC == 64, "the index math below assumes these");

// round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Zero the bf16 elements at positions >= valid of a 16-byte piece.
__device__ __forceinline__ uint4 mask_tail(uint4 v, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int d = 0; d < 4; ++d)
    w[d] &= (2 * d < valid ? 0x0000ffffu : 0u) | (2 * d + 1 < valid ? 0xffff0000u : 0u);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Store n (<= 8) bf16 values: one 16-byte store when whole and aligned,
// element stores otherwise.
__device__ __forceinline__ void store8(uint16_t *dst, uint4 w, int n) {
  if (n == 8 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
    *reinterpret_cast<uint4 *>(dst) = w;
  } else {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    for (int e = 0; e < n; ++e) dst[e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
  }
}

// One chunk of a row-major bf16 matrix: rows row0 .. row0 + 16 NP - 1 (those
// below nrows), columns col0 .. col0+127 (those below ncols, the rest zero).
// Thread t loads 16-byte pieces c = t + 256 q (q < NP): row c / 16, columns
// 8 (c % 16) .. +7.  A piece that starts below ncols stays inside the row:
// ld is a multiple of 8 and at least ncols.
template <int NP>
__device__ __forceinline__ void load_chunk(uint4 (&v)[NP], const uint16_t *base, int64_t ld, int64_t row0,
                                           int64_t nrows, int64_t col0, int64_t ncols) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int c = t + NTHR * q;
    const int64_t r = row0 + (c >> 4);
    const int64_t k = col0 + 8 * (c & 15);
    uint4 x = make_uint4(0, 0, 0, 0);
    if (r < nrows && k < ncols) {
      x = *reinterpret_cast<const uint4 *>(base + r * ld + k);
      if (ncols - k < 8) x = mask_tail(x, (int)(ncols - k));
    }
    v[q] = x;
  }
}

template <int NP>
__device__ __forceinline__ void stage_chunk(char *buf, const uint4 (&v)[NP]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int c = t + NTHR * q;
    *reinterpret_cast<uint4 *>(buf + (c >> 4) * (SROW * 2) + (c & 15) * 16) = v[q];
  }
}

// bf16 MFMA operand: 8 elements of staged row `row` at K offset 16 kk + 8 lg
__device__ __forceinline__ bf16x8 sfrag(const char *buf, int row, int kk, int lg) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(buf + row * (SROW * 2) + (16 * kk + 8 * lg) * 2));
}

// fp32 MFMA operands: 4 elements of row `row` at K offset 8 kb + 4 lg
__device__ __forceinline__ float4 ffrag(const float *M, int row, int kb, int lg) {
  return *reinterpret_cast<const float4 *>(M + row * FROW + 8 * kb + 4 * lg);
}

__device__ __forceinline__ void zero(f32x16 (&a)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) a[i][v] = 0.f;
}

// acc[I] += L[32 I .. 32 I + 31, :] * S[:, 32 w .. 32 w + 31] with L and S
// both in LDS (S read along its rows: exactly symmetric)
__device__ __forceinline__ void mm_lds_lds(f32x16 (&acc)[4], const float *L, const float *S, int w, int lr, int lg) {
#pragma unroll 4
  for (int kb = 0; kb < HM / 8; ++kb) {
    const float4 b = ffrag(S, 32 * w + lr, kb, lg);
    float4 a[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) a[I] = ffrag(L, 32 * I + lr, kb, lg);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].x, b.x, acc[I], 0, 0, 0);
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].y, b.y, acc[I], 0, 0, 0);
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].z, b.z, acc[I], 0, 0, 0);
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].w, b.w, acc[I], 0, 0, 0);
    }
  }
}

// acc[I] += L[32 I .., :] * B with B's column block w in registers: tile K
// of B (rows 32 K ..) register 4 q + e holds row 8 (4 K + q) + 4 lg + e
__device__ __forceinline__ void mm_lds_reg(f32x16 (&acc)[4], const float *L, const f32x16 (&B)[4], int lr, int lg) {
#pragma unroll
  for (int kb = 0; kb < HM / 8; ++kb) {
    float4 a[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) a[I] = ffrag(L, 32 * I + lr, kb, lg);
    const int K = kb >> 2, q = kb & 3;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].x, B[K][4 * q + 0], acc[I], 0, 0, 0);
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].y, B[K][4 * q + 1], acc[I], 0, 0, 0);
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].z, B[K][4 * q + 2], acc[I], 0, 0, 0);
      acc[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[I].w, B[K][4 * q + 3], acc[I], 0, 0, 0);
    }
  }
}

// Row of register r of an accumulator tile (rows 32 I ..): 32 I + rrow(r, lg)
__device__ __forceinline__ int rrow(int r, int lg) { return (r & 3) + 8 * (r >> 2) + 4 * lg; }

// Write column block w (tiles (I, w)) of a symmetric fp32 matrix into LDS so
// that the stored matrix is exactly symmetric: tile (I, w) with I < w and the
// upper triangle of the diagonal tile, each value to (i, j) and (j, i).
__device__ __forceinline__ void put_sym_f32(float *M, const f32x16 (&v)[4], int w, int lr, int lg) {
  const int j = 32 * w + lr;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    if (I > w) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * I + rrow(r, lg);
      if (I == w && i > j) continue;
      M[i * FROW + j] = v[I][r];
      M[j * FROW + i] = v[I][r];
    }
  }
}

// The same for the bf16 pair hi = bf16(v), lo = bf16(v - hi) in two
// staging-layout buffers (rows of SROW).
__device__ __forceinline__ void put_sym_pair(char *hbuf, char *lbuf, const f32x16 (&v)[4], int w, int lr, int lg) {
  uint16_t *H = reinterpret_cast<uint16_t *>(hbuf);
  uint16_t *L = reinterpret_cast<uint16_t *>(lbuf);
  const int j = 32 * w + lr;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    if (I > w) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * I + rrow(r, lg);
      if (I == w && i > j) continue;
      const float x = v[I][r];
      const uint16_t h = (uint16_t)pk2(x, 0.f);
      const uint16_t l = (uint16_t)pk2(x - __uint_as_float((uint32_t)h << 16), 0.f);
      H[i * SROW + j] = h;
      H[j * SROW + i] = h;
      L[i * SROW + j] = l;
      L[j * SROW + i] = l;
    }
  }
}

// Store the output of one 64-row chunk of X^T (rows n0 .. n0+63 of n) into
// U: a wide block's U is Y (m x n, row-major) and comes from the staging
// `rows_j` (staged row j = row j of Y, OROW apart); a tall block's U is Y^T
// (n x m) and comes from `rows_n` (staged row r = row n0 + r of Y^T, SROW
// apart).  16-byte pieces, element stores at ragged or unaligned edges.
__device__ __forceinline__ void store_out(uint16_t *U, int64_t ldu, bool tall, int m, int64_t n, int64_t n0,
                                          const char *rows_j, const char *rows_n) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int cc = tid + NTHR * qq;
    if (!tall) {
      // U row pr (< m), columns n0 + pc8 .. (< n): 8 pieces per staged row
      const int pr = cc >> 3, pc8 = 8 * (cc & 7);
      const uint4 val = *reinterpret_cast<const uint4 *>(rows_j + (pr * OROW + pc8) * 2);
      const int64_t col = n0 + pc8;
      if (pr < m && col < n) store8(U + pr * ldu + col, val, (int)min<int64_t>(n - col, 8));
    } else {
      // U row n0 + pr (< n), columns pc8 .. (< m): 16 pieces per staged row
      const int pr = cc >> 4, pc8 = 8 * (cc & 15);
      const uint4 val = *reinterpret_cast<const uint4 *>(rows_n + (pr * SROW + pc8) * 2);
      const int64_t row = n0 + pr;
      if (row < n && pc8 < m) store8(U + row * ldu + pc8, val, min(m - pc8, 8));
    }
  }
}

// Row block w (tiles (w, J)) of a symmetric matrix, times sc, rounded to
// bf16 into a staging-layout buffer so that the stored matrix is exactly
// symmetric: tiles J > w and the upper triangle of (w, w), each value to
// (i, j) and (j, i).
__device__ __forceinline__ void put_rows_bf16(char *buf, const f32x16 (&v)[4], float sc, int w, int lr, int lg) {
  uint16_t *M = reinterpret_cast<uint16_t *>(buf);
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J < w) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * w + rrow(r, lg), j = 32 * J + lr;
      if (J == w && i > j) continue;
      const uint16_t h = (uint16_t)pk2(v[J][r] * sc, 0.f);
      M[i * SROW + j] = h;
      M[j * SROW + i] = h;
    }
  }
}

// acc[J] = X[32 w .., :] X[32 J .., :]^T over all n columns of the m x n
// row-major bf16 X (rows >= m zero), streaming 128-column chunks through the
// two staging buffers (two chunks in flight in registers).  Ends with a
// barrier: the buffers are free on return.
__device__ __forceinline__ void gram_stream(f32x16 (&acc)[4], const uint16_t *X, int64_t ldx, int m, int64_t n,
                                            char *sb0, char *sb1) {
  const int w = threadIdx.x >> 6, lr = threadIdx.x & 31, lg = (threadIdx.x >> 5) & 1;
  char *sb[2] = {sb0, sb1};
  const int nc = (int)((n + KC - 1) / KC);
  uint4 va[8], vb[8];
  zero(acc);
  auto body = [&](int c, uint4 (&freeset)[8], const uint4 (&held)[8]) {
    if (c + 2 < nc) load_chunk(freeset, X, ldx, 0, m, (int64_t)(c + 2) * KC, n);
    const char *buf = sb[c & 1];
#pragma unroll
    for (int kk = 0; kk < KC / 16; ++kk) {
      const bf16x8 a = sfrag(buf, 32 * w + lr, kk, lg);
#pragma unroll
      for (int J = 0; J < 4; ++J)
        acc[J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sfrag(buf, 32 * J + lr, kk, lg), acc[J], 0, 0, 0);
    }
    if (c + 1 < nc) stage_chunk(sb[(c + 1) & 1], held);
    __syncthreads();
  };
  load_chunk(va, X, ldx, 0, m, 0, n);
  if (nc > 1) load_chunk(vb, X, ldx, 0, m, KC, n);
  stage_chunk(sb[0], va);
  __syncthreads();
  for (int c = 0; c < nc; c += 2) {
    body(c, va, vb);
    if (c + 1 < nc) body(c + 1, vb, va);
  }
}

__global__ __launch_bounds__(NTHR, 1) void ns_head_gram(HeadArgs args) {
  if (args.skip && *args.skip) return;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const TileDev tile = args.tiles[blockIdx.x];
  const ProbDev &P = args.probs[tile.prob];
  const int m = P.m;
  const int64_t n = P.n;
  if (m < 1 || m > HM) return;  // the planner sends only blocks with m <= 128
  const uint16_t *X = reinterpret_cast<const uint16_t *>(args.ws + P.off[R_XR0]);
  const uint16_t *Z = reinterpret_cast<const uint16_t *>(args.ws + P.off[R_XC0]);
  uint16_t *U = reinterpret_cast<uint16_t *>(args.ws + P.off[R_U]);
  const int64_t ldx = P.ld[R_XR0], ldz = P.ld[R_XC0], ldu = P.ld[R_U];
  const bool tall = (P.flags & PF_TALL) != 0;
  const float s = args.scales[tile.prob];
  const int T = args.steps;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  char *sb[2] = {lds, lds + SBUF};   // phase 1: input staging
  float *Rm = reinterpret_cast<float *>(lds);          // phase 2
  float *Pm = reinterpret_cast<float *>(lds + FMAT);
  char *qh = lds, *ql = lds + SBUF;  // phase 3: Q_hi, Q_lo
  char *yb[2] = {lds + Y_IN, lds + Y_IN + YC * SROW * 2};
  char *ob = lds + Y_OUT;

  // ---- 1. R = s^2 X0 X0^T: wave w accumulates tiles (w, J)
  f32x16 racc[4];
  gram_stream(racc, X, ldx, m, n, sb[0], sb[1]);
  // the loop ended with a barrier: the staging buffers are free
  {
    const float sc = s * s;
    const int j0 = lr;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J < w) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * w + rrow(r, lg), j = 32 * J + j0;
        if (J == w && i > j) continue;
        const float v = racc[J][r] * sc;
        Rm[i * FROW + j] = v;
        Rm[j * FROW + i] = v;
      }
    }
  }
  __syncthreads();

  // ---- 2. the chain
  f32x16 q[4], pc[4];
  for (int k = 1; k <= T; ++k) {
    // P = a I + b R + c R R, column block w
    zero(pc);
    mm_lds_lds(pc, Rm, Rm, w, lr, lg);
    {
      const int j = 32 * w + lr;
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // R[i][j] for the four rows of register group g, read along row j
          const float4 rv = ffrag(Rm, j, 4 * I + g, lg);
          const float rr[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 32 * I + 8 * g + 4 * lg + e;
            float x = pc[I][4 * g + e] * args.c;
            x = fmaf(args.b, rr[e], x);
            if (i == j && i < m) x += args.a;
            pc[I][4 * g + e] = x;
          }
        }
    }
    put_sym_f32(Pm, pc, w, lr, lg);
    __syncthreads();
    // Q <- P Q (the first P is Q)
    if (k == 1) {
#pragma unroll
      for (int I = 0; I < 4; ++I) q[I] = pc[I];
    } else {
      f32x16 qn[4];
      zero(qn);
      mm_lds_reg(qn, Pm, q, lr, lg);
#pragma unroll
      for (int I = 0; I < 4; ++I) q[I] = qn[I];
    }
    if (k < T) {
      // R <- P (R P): T = R P from P's column block, then P T
      f32x16 t1[4], rn[4];
      zero(t1);
      mm_lds_reg(t1, Rm, pc, lr, lg);
      zero(rn);
      mm_lds_reg(rn, Pm, t1, lr, lg);
      __syncthreads();  // every wave is done reading R and P
      put_sym_f32(Rm, rn, w, lr, lg);
      __syncthreads();
    }
  }

  // ---- 3. Y^T = s X0^T (Q_hi + Q_lo), chunks of 64 rows of X0^T: wave w
  // computes rows 32 (w % 2) .. of the chunk, columns 64 (w / 2) .. +63
  __syncthreads();  // every wave is done with P (its Q update)
  put_sym_pair(qh, ql, q, w, lr, lg);
  __syncthreads();
  {
    const int rb = w & 1, J0 = 2 * (w >> 1);
    const int ny = (int)((n + YC - 1) / YC);
    uint4 ya[4], yv[4];
    auto body = [&](int c, uint4 (&freeset)[4], const uint4 (&held)[4]) {
      if (c + 2 < ny) load_chunk<4>(freeset, Z, ldz, (int64_t)(c + 2) * YC, n, 0, m);
      const char *buf = yb[c & 1];
      f32x16 y[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) y[t][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KC / 16; ++kk) {
        const bf16x8 a = sfrag(buf, 32 * rb + lr, kk, lg);
        // B = Q[k][j] for j = 32 J + lr, read along row j (exactly symmetric)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int J = J0 + t;
          y[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sfrag(qh, 32 * J + lr, kk, lg), y[t], 0, 0, 0);
          y[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sfrag(ql, 32 * J + lr, kk, lg), y[t], 0, 0, 0);
        }
      }
      __syncthreads();  // every wave has stored the previous chunk's output
      // y[t] register r: row (of the chunk of X0^T) 32 rb + rrow(r), column 32 (J0 + t) + lr
      uint16_t *oh = reinterpret_cast<uint16_t *>(ob);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = 32 * (J0 + t) + lr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 32 * rb + 8 * g + 4 * lg;
          const uint32_t p01 = pk2(y[t][4 * g] * s, y[t][4 * g + 1] * s);
          const uint32_t p23 = pk2(y[t][4 * g + 2] * s, y[t][4 * g + 3] * s);
          if (!tall) {
            // staged row j of Y, columns r0 .. r0+3 of the chunk
            *reinterpret_cast<uint2 *>(ob + (j * OROW + r0) * 2) = make_uint2(p01, p23);
          } else {
            // staged rows r0 .. r0+3 of Y^T, column j
            oh[(r0 + 0) * SROW + j] = (uint16_t)p01;
            oh[(r0 + 1) * SROW + j] = (uint16_t)(p01 >> 16);
            oh[(r0 + 2) * SROW + j] = (uint16_t)p23;
            oh[(r0 + 3) * SROW + j] = (uint16_t)(p23 >> 16);
          }
        }
      }
      if (c + 1 < ny) stage_chunk<4>(yb[(c + 1) & 1], held);
      __syncthreads();
      store_out(U, ldu, tall, m, n, (int64_t)c * YC, ob, ob);
    };
    load_chunk<4>(ya, Z, ldz, 0, n, 0, m);
    if (ny > 1) load_chunk<4>(yv, Z, ldz, YC, n, 0, m);
    stage_chunk<4>(yb[0], ya);
    __syncthreads();
    for (int c = 0; c < ny; c += 2) {
      body(c, ya, yv);
      if (c + 1 < ny) body(c + 1, yv, ya);
    }
  }
}


// Standard form, T >= 1 steps, on the same blocks:
//   A0 = s^2 X0 X0^T (streaming X0, as R above), then per step t:
//   C = a I + b A + c A A (bf16 MFMA on the bf16 A; C stored bf16), and over
//   64-row chunks of Z = X^T (n x m): Z' = s_t Z C (C symmetric, so this is
//   (s_t C X)^T), rounded to bf16 and staged in both orientations; A' =
//   Z'^T Z' accumulated from the staged bf16 chunk (the next step's A, the
//   product of the stored X' with itself), and Z' written back over Z in
//   place (each chunk's rows are read before they are written, by this
//   workgroup alone); at the last step the chunk goes to U instead.
// s_0 = s (the norm folded into the first products), s_t = 1 after.  The
// rounding points are those of the tiled path: A, C and X bf16.
constexpr int SD_A = 0, SD_C = SBUF, SD_IN = 2 * SBUF;
constexpr int SD_S1 = SD_IN + 2 * YC * SROW * 2;   // Z'^T chunk: [j][r], OROW apart
constexpr int SD_S2 = SD_S1 + OBUF;                // Z' chunk: [r][j], SROW apart
constexpr int SD_BYTES = SD_S2 + YC * SROW * 2;    // 140288
static_assert(SD_BYTES <= 160 * 1024, "the standard kernel's LDS fits the CU");

__global__ __launch_bounds__(NTHR, 1) void ns_head_std(HeadArgs args) {
  if (args.skip && *args.skip) return;
  __shared__ __attribute__((aligned(16))) char lds[SD_BYTES];
  const TileDev tile = args.tiles[blockIdx.x];
  const ProbDev &P = args.probs[tile.prob];
  const int m = P.m;
  const int64_t n = P.n;
  if (m < 1 || m > HM) return;  // the planner sends only blocks with m <= 128
  const uint16_t *X = reinterpret_cast<const uint16_t *>(args.ws + P.off[R_XR0]);
  uint16_t *Zw = reinterpret_cast<uint16_t *>(args.ws + P.off[R_XC0]);
  uint16_t *U = reinterpret_cast<uint16_t *>(args.ws + P.off[R_U]);
  const int64_t ldx = P.ld[R_XR0], ldz = P.ld[R_XC0], ldu = P.ld[R_U];
  const bool tall = (P.flags & PF_TALL) != 0;
  const float s = args.scales[tile.prob];
  const int T = args.steps;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  char *Ab = lds + SD_A, *Cb = lds + SD_C;
  char *yb[2] = {lds + SD_IN, lds + SD_IN + YC * SROW * 2};
  char *s1 = lds + SD_S1, *s2 = lds + SD_S2;

  // ---- A0 = s^2 X0 X0^T (its staging uses the space of A and C)
  f32x16 aacc[4];
  gram_stream(aacc, X, ldx, m, n, lds, lds + SBUF);
  put_rows_bf16(Ab, aacc, s * s, w, lr, lg);
  __syncthreads();

  const int ny = (int)((n + YC - 1) / YC);
  const int rb = w & 1, J0 = 2 * (w >> 1);
  for (int t = 0; t < T; ++t) {
    const bool last = t == T - 1;
    const float st = t == 0 ? s : 1.f;
    // C = a I + b A + c A A: row block w, exactly symmetric (B = A[k][j]
    // read along row j)
    {
      f32x16 cacc[4];
      zero(cacc);
#pragma unroll
      for (int kk = 0; kk < HM / 16; ++kk) {
        const bf16x8 a = sfrag(Ab, 32 * w + lr, kk, lg);
#pragma unroll
        for (int J = 0; J < 4; ++J)
          cacc[J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sfrag(Ab, 32 * J + lr, kk, lg), cacc[J], 0, 0, 0);
      }
      uint16_t *Ch = reinterpret_cast<uint16_t *>(Cb);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J < w) continue;
        const int j = 32 * J + lr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i0 = 32 * w + 8 * g + 4 * lg;
          // A[i0 .. i0+3][j], read along row j
          const uint2 av = *reinterpret_cast<const uint2 *>(Ab + (j * SROW + i0) * 2);
          const float ad[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                               __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            if (J == w && i > j) continue;
            float x = cacc[J][4 * g + e] * args.c;
            x = fmaf(args.b, ad[e], x);
            if (i == j && i < m) x += args.a;
            const uint16_t h = (uint16_t)pk2(x, 0.f);
            Ch[i * SROW + j] = h;
            Ch[j * SROW + i] = h;
          }
        }
      }
    }
    __syncthreads();

    zero(aacc);
    uint4 ya[4], yv[4];
    auto body = [&](int c, uint4 (&freeset)[4], const uint4 (&held)[4]) {
      if (c + 2 < ny) load_chunk<4>(freeset, Zw, ldz, (int64_t)(c + 2) * YC, n, 0, m);
      const char *buf = yb[c & 1];
      f32x16 y[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int v = 0; v < 16; ++v) y[t2][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KC / 16; ++kk) {
        const bf16x8 a = sfrag(buf, 32 * rb + lr, kk, lg);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          y[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sfrag(Cb, 32 * (J0 + t2) + lr, kk, lg), y[t2], 0, 0, 0);
      }
      __syncthreads();  // every wave is done with the previous chunk's staging
      uint16_t *s2h = reinterpret_cast<uint16_t *>(s2);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int j = 32 * (J0 + t2) + lr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 32 * rb + 8 * g + 4 * lg;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = y[t2][4 * g + e] * 1.f;
            x *= st;
            v[e] = x;
          }
          const uint32_t p01 = pk2(v[0], v[1]), p23 = pk2(v[2], v[3]);
          *reinterpret_cast<uint2 *>(s1 + (j * OROW + r0) * 2) = make_uint2(p01, p23);
          s2h[(r0 + 0) * SROW + j] = (uint16_t)p01;
          s2h[(r0 + 1) * SROW + j] = (uint16_t)(p01 >> 16);
          s2h[(r0 + 2) * SROW + j] = (uint16_t)p23;
          s2h[(r0 + 3) * SROW + j] = (uint16_t)(p23 >> 16);
        }
      }
      if (c + 1 < ny) stage_chunk<4>(yb[(c + 1) & 1], held);
      __syncthreads();
      const int64_t n0 = (int64_t)c * YC;
      if (!last) {
        // A' += Z'c^T Z'c: row block w, K = the chunk's 64 rows
#pragma unroll
        for (int kk = 0; kk < YC / 16; ++kk) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4 *>(s1 + ((32 * w + lr) * OROW + 16 * kk + 8 * lg) * 2));
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const bf16x8 b = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(s1 + ((32 * J + lr) * OROW + 16 * kk + 8 * lg) * 2));
            aacc[J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, aacc[J], 0, 0, 0);
          }
        }
        // Z' rows back over Z: row n0 + pr (< n), columns pc8 .. (< m)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int cc = tid + NTHR * qq;
          const int pr = cc >> 4, pc8 = 8 * (cc & 15);
          const int64_t row = n0 + pr;
          if (row < n && pc8 < m)
            store8(Zw + row * ldz + pc8, *reinterpret_cast<const uint4 *>(s2 + (pr * SROW + pc8) * 2),
                   min(m - pc8, 8));
        }
      } else {
        store_out(U, ldu, tall, m, n, n0, s1, s2);
      }
    };
    load_chunk<4>(ya, Zw, ldz, 0, n, 0, m);
    if (ny > 1) load_chunk<4>(yv, Zw, ldz, YC, n, 0, m);
    stage_chunk<4>(yb[0], ya);
    __syncthreads();
    for (int c = 0; c < ny; c += 2) {
      body(c, ya, yv);
      if (c + 1 < ny) body(c + 1, yv, ya);
    }
    if (!last) {
      // the next step's A; A was last read for this step's C (barriers since)
      put_rows_bf16(Ab, aacc, 1.f, w, lr, lg);
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_head(const HeadArgs &a, int nprob, hipStream_t s) {
  if (nprob <= 0) return hipSuccess;
  if (a.standard) hipLaunchKernelGGL(ns_head_std, dim3(nprob), dim3(NTHR), 0, s, a);
  else hipLaunchKernelGGL(ns_head_gram, dim3(nprob), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
