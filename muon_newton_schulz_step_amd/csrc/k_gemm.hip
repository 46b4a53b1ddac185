// Grouped Newton-Schulz GEMMs on gfx950 MFMA.
//
// Every product of the iteration is written as C = A B^T with both operands
// row-major and K contiguous ("NT"): X X^T, A A (A symmetric), B X (X^T is
// kept as its own buffer), and in the Gram form R R, P Q, P R, (PR) P (all
// polynomials in X0 X0^T, hence symmetric and commuting).  One launch covers
// every problem of the group through a tile list; symmetric outputs list only
// tiles with tm <= tn and write the mirror tile from the same accumulators.
//
// The epilogue fuses the quintic: C = s^p (cd D + cacc acc) + cdiag I, where
// D is a second operand read in the epilogue (A for bA + cA^2, X for
// aX + BX, R for aI + bR + cR^2) and s is the block's 1/(||u|| + eps), so the
// normalisation is folded into the first products instead of a separate pass.
//
// Tiles: 128 x 128 outputs per 256-thread workgroup (4 wave64s as 2 x 2, each
// 64 x 64 = 2 x 2 MFMA 32x32 blocks), K staged through LDS in 64-byte rows
// (32 bf16 or 16 fp32) padded to 80 bytes, which keeps every 16-byte
// fragment read conflict-free; the next K tile is prefetched to registers
// while the current one feeds the MFMAs (double-buffered LDS).
#include <hip/hip_runtime.h>

#include "elem.hpp"
#include "tables.hpp"

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int BM = GEMM_TILE, BN = GEMM_TILE;
constexpr int ROWB = 80;           // LDS bytes per staged row (64 + 16 pad)
constexpr int OPB = BM * ROWB;     // LDS bytes per operand tile
constexpr int NTHR = 256;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)f, (__bf16)0.f};
  return (uint16_t)__builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void store_elem(char *base, int64_t idx, float v, bool f32) {
  if (f32) reinterpret_cast<float *>(base)[idx] = v;
  else reinterpret_cast<uint16_t *>(base)[idx] = f2bf(v);
}

__device__ __forceinline__ float load_elem(const char *base, int64_t idx, bool f32) {
  return f32 ? reinterpret_cast<const float *>(base)[idx] : bf2f(reinterpret_cast<const uint16_t *>(base)[idx]);
}

// Zero the elements at positions >= valid of a 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ uint4 mask_tail(uint4 v, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (BF16) {
      uint32_t keep = (2 * d < valid ? 0x0000ffffu : 0u) | (2 * d + 1 < valid ? 0xffff0000u : 0u);
      w[d] &= keep;
    } else {
      if (d >= valid) w[d] = 0u;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// store n (<= 8) bf16 values packed in w at dst: one 16-byte store when
// whole and aligned, element stores otherwise
__device__ __forceinline__ void store8(uint16_t *dst, uint4 w, int n) {
  if (n == 8 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
    *reinterpret_cast<uint4 *>(dst) = w;
  } else {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    for (int e = 0; e < n; ++e) dst[e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
  }
}

// Epilogue for bf16 outputs (and, if any, a bf16 symmetric D): the
// accumulators are transformed in registers (D read as D[col][row .. row+3],
// which its symmetry allows), staged once as bf16 in column-major order
// (column stride 264 bytes) behind one barrier, then stored 16 bytes per
// lane: row-major outputs gathered with transposing LDS reads
// (ds_read_b64_tr_b16: lane i of a 16-lane group receives element (i % 4) of
// the 8 bytes lane 4 e + i / 4 addresses, for e = 0..3), transposed and
// mirror outputs with contiguous reads.
constexpr int SCB = 264;
__device__ __forceinline__ void staged_epilogue(const GemmArgs &args, const GemmRecipe &R, const ProbDev &P,
                                                const TileDev &tile, const f32x16 (&acc)[2][2], float sc,
                                                bool mirror, bool t0, bool t1, bool diag, const char *D,
                                                int64_t ldd, char *S0, int64_t ld0, char *S1, int64_t ld1,
                                                int64_t M, int64_t N, int64_t m0, int64_t n0, char *lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t col0 = n0 + wn * 64 + lr;       // + 32 j
  const int64_t row0 = m0 + wm * 64 + 4 * lg;   // + 32 i + 8 g
  uint2 dq[2][2][4];
  if (D) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t gj = col0 + 32 * j, gi = row0 + 32 * i + 8 * g;
          uint2 w = make_uint2(0, 0);
          // rows gi .. gi+3 may run past M only where nothing is stored
          if (gj < N && gi < M) w = *reinterpret_cast<const uint2 *>(D + (gj * ldd + gi) * 2);
          dq[i][j][g] = w;
        }
  }
  __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t gi = row0 + 32 * i + 8 * g, gj = col0 + 32 * j;
        float d[4] = {0.f, 0.f, 0.f, 0.f};
        if (D) {
          const uint2 w = dq[i][j][g];
          d[0] = __uint_as_float(w.x << 16); d[1] = __uint_as_float(w.x & 0xffff0000u);
          d[2] = __uint_as_float(w.y << 16); d[3] = __uint_as_float(w.y & 0xffff0000u);
        }
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = acc[i][j][4 * g + e] * R.cacc;
          if (D) x = fmaf(R.cd, d[e], x);
          x *= sc;
          if (diag && gi + e == gj) x += R.cdiag;
          h[e] = f2bf(x);
        }
        const int cl = wn * 64 + 32 * j + lr, rl = wm * 64 + 32 * i + 8 * g + 4 * lg;
        *reinterpret_cast<uint2 *>(lds + cl * SCB + rl * 2) =
            make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
      }
  __syncthreads();
  const bool r0 = !t0, r1 = S1 && !t1, c0 = t0 || mirror, c1 = S1 && (t1 || mirror);
  char *rowA = r0 ? S0 : S1, *rowB = S1;
  const int64_t rowLA = r0 ? ld0 : ld1, rowLB = ld1;
  const int nrow = (int)r0 + (int)r1;
  char *colA = c0 ? S0 : S1, *colB = S1;
  const int64_t colLA = c0 ? ld0 : ld1, colLB = ld1;
  const int ncol = (int)c0 + (int)c1;
  if (nrow) {
    // 16-lane group q4 of wave w, step it: rows rb .. rb+16 with
    // rb = 16 (4 (it / 4) + w), columns cb .. cb+8 with cb = 32 (it % 4) +
    // 8 q4; lane li supplies column cb + li/4 (and +4), rows rb + 4 (li % 4)
    // .. +3, and ends up with columns cb .. cb+7 of row rb + li
    const int q4 = lane >> 4, li = lane & 15;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int rb = 16 * (4 * (it >> 2) + wave);
      const int cb = 32 * (it & 3) + 8 * q4;
      const char *base = lds + (cb + (li >> 2)) * SCB + (rb + 4 * (li & 3)) * 2;
      const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base));
      const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + 4 * SCB));
      // the reads exchange data across the 16 lanes of a group: keep them
      // ahead of the per-lane branch below, with every lane active
      asm volatile("" ::"v"(lo4), "v"(hi4));
      const int64_t gi = m0 + rb + li, gj = n0 + cb;
      if (gi >= M || gj >= N) continue;
      const uint4 w = make_uint4((uint32_t)(uint16_t)lo4[0] | ((uint32_t)(uint16_t)lo4[1] << 16),
                                 (uint32_t)(uint16_t)lo4[2] | ((uint32_t)(uint16_t)lo4[3] << 16),
                                 (uint32_t)(uint16_t)hi4[0] | ((uint32_t)(uint16_t)hi4[1] << 16),
                                 (uint32_t)(uint16_t)hi4[2] | ((uint32_t)(uint16_t)hi4[3] << 16));
      const int nv = (int)min<int64_t>(N - gj, 8);
      store8(reinterpret_cast<uint16_t *>(rowA) + gi * rowLA + gj, w, nv);
      if (nrow > 1) store8(reinterpret_cast<uint16_t *>(rowB) + gi * rowLB + gj, w, nv);
    }
  }
  if (ncol) {
    // 16 lanes per column: column c, rows 8 (lane % 16) .. +8
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int c = 4 * (4 * it + wave) + (lane >> 4);
      const int r8 = 8 * (lane & 15);
      const char *src = lds + c * SCB + r8 * 2;
      const uint2 a2 = *reinterpret_cast<const uint2 *>(src);
      const uint2 b2 = *reinterpret_cast<const uint2 *>(src + 8);
      const int64_t gj = n0 + c, gi = m0 + r8;
      if (gj >= N || gi >= M) continue;
      const uint4 w = make_uint4(a2.x, a2.y, b2.x, b2.y);
      const int nv = (int)min<int64_t>(M - gi, 8);
      store8(reinterpret_cast<uint16_t *>(colA) + gj * colLA + gi, w, nv);
      if (ncol > 1) store8(reinterpret_cast<uint16_t *>(colB) + gj * colLB + gi, w, nv);
    }
  }
  (void)args; (void)P; (void)tile;
}

template <bool BF16>
__global__ __launch_bounds__(NTHR, 3) void ns_gemm(GemmArgs args) {
  if (args.skip && *args.skip) return;
  constexpr int ES = BF16 ? 2 : 4;   // operand element bytes
  constexpr int BK = 64 / ES;        // K elements per staged row
  constexpr int EPC = 16 / ES;       // elements per 16-byte chunk
  __shared__ __attribute__((aligned(16))) char lds[2][2][OPB];

  const TileDev tile = args.tiles[blockIdx.x];
  const ProbDev &P = args.probs[tile.prob];
  const GemmRecipe R = args.r;
  const int64_t M = R.dimM ? P.n : P.m;
  const int64_t N = R.dimN ? P.n : P.m;
  const int64_t K = R.dimK ? P.n : P.m;
  const char *A = args.ws + P.off[R.rA];
  const char *B = args.ws + P.off[R.rB];
  const int64_t lda = P.ld[R.rA], ldb = P.ld[R.rB];
  const int64_t m0 = (int64_t)tile.tm * BM, n0 = (int64_t)tile.tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;

  uint4 ra[2], rb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = tid + NTHR * q;
      const int row = c >> 2, kc = c & 3;
      const int64_t gk = (int64_t)kt * BK + kc * EPC;
      const int valid = (int)min<int64_t>(K - gk, (int64_t)EPC);
      uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
      if (valid > 0) {
        const int64_t ga = m0 + row, gb = n0 + row;
        if (ga < M) {
          va = *reinterpret_cast<const uint4 *>(A + (ga * lda + gk) * ES);
          if (valid < EPC) va = mask_tail<BF16>(va, valid);
        }
        if (gb < N) {
          vb = *reinterpret_cast<const uint4 *>(B + (gb * ldb + gk) * ES);
          if (valid < EPC) vb = mask_tail<BF16>(vb, valid);
        }
      }
      ra[q] = va;
      rb[q] = vb;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = tid + NTHR * q;
      const int row = c >> 2, kc = c & 3;
      *reinterpret_cast<uint4 *>(&lds[buf][0][row * ROWB + kc * 16]) = ra[q];
      *reinterpret_cast<uint4 *>(&lds[buf][1][row * ROWB + kc * 16]) = rb[q];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (int)((K + BK - 1) / BK);
  gload(0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const uint4 *>(&lds[buf][0][(wm * 64 + i * 32 + lr) * ROWB + ks * 32 + lg * 16]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const uint4 *>(&lds[buf][1][(wn * 64 + j * 32 + lr) * ROWB + ks * 32 + lg * 16]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (BF16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[i]),
                                                                __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(fa[i].x), __uint_as_float(fb[j].x),
                                                             acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(fa[i].y), __uint_as_float(fb[j].y),
                                                             acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(fa[i].z), __uint_as_float(fb[j].z),
                                                             acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(fa[i].w), __uint_as_float(fb[j].w),
                                                             acc[i][j], 0, 0, 0);
          }
        }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue
  float sc = 1.f;
  if (R.scale_pow) {
    const float s = args.scales[tile.prob];
    sc = R.scale_pow == 2 ? s * s : s;
  }
  const bool mirror = (R.flags & GF_SYM) && tile.tm != tile.tn;
  const bool t0 = (R.flags & GF_S0_TRANS) || ((R.flags & GF_S0_PROBT) && (P.flags & PF_TALL));
  const bool t1 = (R.flags & GF_S1_TRANS) != 0;
  const bool f0 = (R.flags & GF_S0_F32) != 0, f1 = (R.flags & GF_S1_F32) != 0, fd = (R.flags & GF_D_F32) != 0;
  const bool diag = (R.flags & GF_DIAG) != 0;
  const char *D = R.rD >= 0 ? args.ws + P.off[R.rD] : nullptr;
  const int64_t ldd = R.rD >= 0 ? P.ld[R.rD] : 0;
  char *S0 = args.ws + P.off[R.rS0];
  const int64_t ld0 = P.ld[R.rS0];
  char *S1 = R.rS1 >= 0 ? args.ws + P.off[R.rS1] : nullptr;
  const int64_t ld1 = R.rS1 >= 0 ? P.ld[R.rS1] : 0;
  if (!f0 && (!S1 || !f1) && (!D || (!fd && (R.flags & GF_SYM)))) {
    staged_epilogue(args, R, P, tile, acc, sc, mirror, t0, t1, diag, D, ldd, S0, ld0, S1, ld1, M, N, m0, n0,
                    &lds[0][0][0]);
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gi = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
        const int64_t gj = n0 + wn * 64 + j * 32 + lr;
        if (gi < M && gj < N) {
          float val = acc[i][j][v] * R.cacc;
          if (D) val = fmaf(R.cd, load_elem(D, gi * ldd + gj, fd), val);
          val *= sc;
          if (diag && gi == gj) val += R.cdiag;
          store_elem(S0, t0 ? gj * ld0 + gi : gi * ld0 + gj, val, f0);
          if (mirror) store_elem(S0, gj * ld0 + gi, val, f0);
          if (S1) {
            store_elem(S1, t1 ? gj * ld1 + gi : gi * ld1 + gj, val, f1);
            if (mirror) store_elem(S1, gj * ld1 + gi, val, f1);
          }
        }
      }
}

}  // namespace

hipError_t launch_gemm(bool bf16_operands, const GemmArgs &a, int ntiles, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  if (bf16_operands) hipLaunchKernelGGL(ns_gemm<true>, dim3(ntiles), dim3(NTHR), 0, s, a);
  else hipLaunchKernelGGL(ns_gemm<false>, dim3(ntiles), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
