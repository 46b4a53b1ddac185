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

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
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

template <bool BF16>
__global__ __launch_bounds__(NTHR) void ns_gemm(GemmArgs args) {
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
