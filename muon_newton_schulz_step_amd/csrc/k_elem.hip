// HBM-bound kernels of the Muon step on gfx950:
//   K0  fp32 gradient accumulation over micro-batches
//   K1  fp32 momentum lerp + Nesterov blend + per-block sum of squares +
//       the block's two copies (original layout and transposed) in the
//       Newton-Schulz operand dtype
//   KN  per-block norm finalisation (fixed-order reduction of K1 partials)
//   K3  shape scale + owned-run scatter into the fp32 flat partitions
//   KC  zero-step output (the normalised input itself)
// Every reduction has a fixed order and no float atomics, so results are
// bitwise reproducible run to run.
#include <hip/hip_runtime.h>

#include "elem.hpp"
#include "tables.hpp"

namespace muon {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quietened).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_as_f32(const void *p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_from_f32(void *p, int64_t i, float v) {
  if constexpr (BF16) static_cast<uint16_t *>(p)[i] = f32_to_bf16(v);
  else static_cast<float *>(p)[i] = v;
}

// Largest index i in [0, n) with key(i) <= t, for a non-decreasing key.
template <class F>
__device__ __forceinline__ int find_owner(int n, int64_t t, F key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (key(mid) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ----------------------------------------------------------------- K0

template <bool GBF16>
__global__ __launch_bounds__(256) void k0_accumulate(const K0Mat *mats, int nmat, int first) {
  const int64_t ch = blockIdx.x;
  const int i = find_owner(nmat, ch, [&](int k) { return mats[k].chunk0; });
  float *acc = mats[i].acc;
  const void *g = mats[i].g;
  const int64_t start = (ch - mats[i].chunk0) * K0_CHUNK;
  const int64_t end = min(start + (int64_t)K0_CHUNK, mats[i].numel);
  for (int64_t j = start + threadIdx.x; j < end; j += 256) {
    float v = load_as_f32<GBF16>(g, j);
    acc[j] = first ? v : acc[j] + v;
  }
}

// ----------------------------------------------------------------- K1

template <bool GBF16>
__global__ __launch_bounds__(256) void k1_momentum(const K1Prob *probs, int nprob, char *ws, float *partials,
                                                   float beta, float omb, int nesterov) {
  __shared__ float tile[K1_TILE][K1_TILE + 1];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int pi = find_owner(nprob, t, [&](int k) { return (int64_t)probs[k].tile0; });
  const K1Prob P = probs[pi];
  const int lt = t - P.tile0;
  const int tr = lt / P.tiles_c, tc = lt - tr * P.tiles_c;
  const int r0 = tr * K1_TILE, c0 = tc * K1_TILE;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  void *orig = ws + P.orig_off;
  void *trans = ws + P.trans_off;
  float ss = 0.f;
  const int64_t c = c0 + tx;
  for (int i = 0; i < 16; ++i) {
    const int r = ty * 16 + i;
    const int64_t gr = r0 + r;
    float u = 0.f;
    if (gr < P.hr && c < P.cols) {
      const int64_t idx = (P.row0 + gr) * P.cols + c;
      const float g = load_as_f32<GBF16>(P.grad, idx);
      const float m = P.mom[idx];
      const float og = omb * g;
      const float mn = fmaf(beta, m, og);
      P.mom[idx] = mn;
      u = nesterov ? fmaf(beta, mn, og) : mn;
      ss = fmaf(u, u, ss);
      if (P.xbf16) store_from_f32<true>(orig, gr * P.orig_ld + c, u);
      else store_from_f32<false>(orig, gr * P.orig_ld + c, u);
    }
    tile[r][tx] = u;
  }
  __syncthreads();
  for (int i = 0; i < 16; ++i) {
    const int cc = ty * 16 + i;
    const int64_t gc = c0 + cc, gr = r0 + tx;
    if (gc < P.cols && gr < P.hr) {
      if (P.xbf16) store_from_f32<true>(trans, gc * P.trans_ld + gr, tile[tx][cc]);
      else store_from_f32<false>(trans, gc * P.trans_ld + gr, tile[tx][cc]);
    }
  }
  // block sum of squares: wave butterfly, then the 4 waves in order
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (tx == 0) red[ty] = ss;
  __syncthreads();
  if (threadIdx.x == 0) partials[t] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ----------------------------------------------------------------- KN

__global__ __launch_bounds__(256) void kn_finalize(const K1Prob *probs, const float *partials, float *scales,
                                                   float eps) {
  __shared__ double red[256];
  const K1Prob P = probs[blockIdx.x];
  double s = 0.0;
  for (int i = threadIdx.x; i < P.ntiles; i += 256) s += (double)partials[P.tile0 + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float nrm = (float)sqrt(red[0]);
    scales[blockIdx.x] = 1.0f / (nrm + eps);
  }
}

// ----------------------------------------------------------------- K3

__global__ __launch_bounds__(256) void k3_scatter(const K3Run *runs, int nrun) {
  const int64_t ch = blockIdx.x;
  const int i = find_owner(nrun, ch, [&](int k) { return runs[k].chunk0; });
  const K3Run R = runs[i];
  const int64_t start = (ch - R.chunk0) * K3_CHUNK;
  const int64_t end = min(start + (int64_t)K3_CHUNK, R.length);
  if (R.src_bf16) {
    for (int64_t j = start + threadIdx.x; j < end; j += 256) R.dst[j] = load_as_f32<true>(R.src, R.first + j) * R.scale;
  } else {
    for (int64_t j = start + threadIdx.x; j < end; j += 256) R.dst[j] = load_as_f32<false>(R.src, R.first + j) * R.scale;
  }
}

// ----------------------------------------------------------------- KC

__global__ __launch_bounds__(256) void kc_copy_scaled(const ProbDev *probs, const K1Prob *k1, char *ws,
                                                      const float *scales) {
  const int p = blockIdx.x;
  const K1Prob K = k1[p];
  const ProbDev D = probs[p];
  const float s = scales[p];
  const void *src = ws + K.orig_off;
  void *dst = ws + D.off[R_U];
  const int64_t n = (int64_t)K.hr * K.cols;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const int64_t r = j / K.cols, c = j - r * K.cols;
    if (K.xbf16) store_from_f32<true>(dst, j, s * load_as_f32<true>(src, r * K.orig_ld + c));
    else store_from_f32<false>(dst, j, s * load_as_f32<false>(src, r * K.orig_ld + c));
  }
}

// ----------------------------------------------------------------- launchers

hipError_t launch_k0(const K0Mat *mats, int nmat, int64_t chunks, bool gbf16, int first, hipStream_t s) {
  if (chunks <= 0) return hipSuccess;
  if (gbf16) hipLaunchKernelGGL(k0_accumulate<true>, dim3((unsigned)chunks), dim3(256), 0, s, mats, nmat, first);
  else hipLaunchKernelGGL(k0_accumulate<false>, dim3((unsigned)chunks), dim3(256), 0, s, mats, nmat, first);
  return hipGetLastError();
}

hipError_t launch_k1(const K1Prob *probs, int nprob, int tiles, char *ws, float *partials, float beta, int nesterov,
                     bool gbf16, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  const float omb = 1.0f - beta;
  dim3 g((unsigned)tiles), b(256);
  if (gbf16) hipLaunchKernelGGL(k1_momentum<true>, g, b, 0, s, probs, nprob, ws, partials, beta, omb, nesterov);
  else hipLaunchKernelGGL(k1_momentum<false>, g, b, 0, s, probs, nprob, ws, partials, beta, omb, nesterov);
  return hipGetLastError();
}

hipError_t launch_kn(const K1Prob *probs, int nprob, const float *partials, float *scales, float eps, hipStream_t s) {
  if (nprob <= 0) return hipSuccess;
  hipLaunchKernelGGL(kn_finalize, dim3(nprob), dim3(256), 0, s, probs, partials, scales, eps);
  return hipGetLastError();
}

hipError_t launch_k3(const K3Run *runs, int nrun, int64_t chunks, hipStream_t s) {
  if (chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k3_scatter, dim3((unsigned)chunks), dim3(256), 0, s, runs, nrun);
  return hipGetLastError();
}

hipError_t launch_kc(const ProbDev *probs, const K1Prob *k1, int nprob, char *ws, const float *scales, hipStream_t s) {
  if (nprob <= 0) return hipSuccess;
  hipLaunchKernelGGL(kc_copy_scaled, dim3(nprob), dim3(256), 0, s, probs, k1, ws, scales);
  return hipGetLastError();
}

}  // namespace muon
