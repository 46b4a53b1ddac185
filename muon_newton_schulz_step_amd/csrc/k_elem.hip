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

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.f); }

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

// 8 consecutive elements -> fp32 (16-byte bf16 load or two 16-byte fp32 loads)
template <bool BF16>
__device__ __forceinline__ void load8(const void *p, int64_t i, float *v) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(x[k] << 16);
      v[2 * k + 1] = __uint_as_float(x[k] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ void store8_f32(float *p, const float *v) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Each workgroup owns K0_CHUNK elements of one matrix; 8 per lane per
// iteration when the chunk is 16-byte aligned on both sides.
template <bool GBF16>
__global__ __launch_bounds__(256) void k0_accumulate(const K0Mat *mats, int nmat, int first) {
  const int64_t ch = blockIdx.x;
  const int i = find_owner(nmat, ch, [&](int k) { return mats[k].chunk0; });
  float *acc = mats[i].acc;
  const void *g = mats[i].g;
  const int64_t start = (ch - mats[i].chunk0) * K0_CHUNK;
  const int64_t end = min(start + (int64_t)K0_CHUNK, mats[i].numel);
  const bool vec = aligned16(acc + start) && aligned16(GBF16 ? (const void *)(static_cast<const uint16_t *>(g) + start)
                                                             : (const void *)(static_cast<const float *>(g) + start));
  int64_t j = start;
  if (vec && end - start == K0_CHUNK) {
    // a whole chunk: two 8-element groups per lane, all loads first
    const int64_t j0 = start + 8 * threadIdx.x, j1 = j0 + 8 * 256;
    float v0[8], v1[8];
    load8<GBF16>(g, j0, v0);
    load8<GBF16>(g, j1, v1);
    if (!first) {
      float a0[8], a1[8];
      load8<false>(acc, j0, a0);
      load8<false>(acc, j1, a1);
#pragma unroll
      for (int k = 0; k < 8; ++k) { v0[k] = a0[k] + v0[k]; v1[k] = a1[k] + v1[k]; }
    }
    store8_f32(acc + j0, v0);
    store8_f32(acc + j1, v1);
    return;
  }
  if (vec) {
    for (j = start + 8 * threadIdx.x; j + 8 <= end; j += 8 * 256) {
      float v[8];
      load8<GBF16>(g, j, v);
      if (!first) {
        float a[8];
        load8<false>(acc, j, a);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = a[k] + v[k];
      }
      store8_f32(acc + j, v);
    }
    j = start + (end - start) / 8 * 8;   // scalar tail
    for (j += threadIdx.x; j < end; j += 256) {
      const float v = load_as_f32<GBF16>(g, j);
      acc[j] = first ? v : acc[j] + v;
    }
    return;
  }
  for (j = start + threadIdx.x; j < end; j += 256) {
    const float v = load_as_f32<GBF16>(g, j);
    acc[j] = first ? v : acc[j] + v;
  }
}

// ----------------------------------------------------------------- K1

// 4 consecutive elements -> fp32 / fp32 -> 4 consecutive elements
template <bool BF16>
__device__ __forceinline__ void load4(const void *p, int64_t i, float *v) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
}

__device__ __forceinline__ void store4(void *p, int64_t i, const float *v, bool bf16) {
  if (bf16) {
    uint2 w;
    w.x = f32x2_to_bf16x2(v[0], v[1]);
    w.y = f32x2_to_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p) + i) = w;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// One 64 x 64 tile of one block per workgroup.  Pass 1: each thread takes
// row quads (4 consecutive columns) of rows ty, ty+16, ty+32, ty+48; vector
// loads/stores when the matrix rows are 16-byte aligned and the quad is
// whole, element accesses otherwise.  Pass 2: the transposed copy, one
// 4-row quad of one column per access, read from the LDS tile.
template <bool GBF16>
__global__ __launch_bounds__(256) void k1_momentum(const K1Prob *probs, int nprob, char *ws, float *partials,
                                                   float beta, float omb, int nesterov, float gs,
                                                   const int32_t *skip) {
  if (skip && *skip) return;
  __shared__ float tile[K1_TILE][K1_TILE + 1];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int pi = find_owner(nprob, t, [&](int k) { return (int64_t)probs[k].tile0; });
  const K1Prob P = probs[pi];
  const int lt = t - P.tile0;
  const int tr = lt / P.tiles_c, tc = lt - tr * P.tiles_c;
  const int r0 = tr * K1_TILE, c0 = tc * K1_TILE;
  void *orig = ws + P.orig_off;
  void *trans = ws + P.trans_off;
  const bool xb = P.xbf16 != 0;
  const bool vec_rows = (P.cols % 4) == 0 && aligned16(P.mom) && ((reinterpret_cast<uintptr_t>(P.grad) & (GBF16 ? 7 : 15)) == 0);
  float ss = 0.f;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int cq = tx * 4;
  const int64_t c = c0 + cq;
  auto one = [&](float g, float m, float &mn, float &u) {
    const float og = omb * (g * gs);
    mn = fmaf(beta, m, og);
    u = nesterov ? fmaf(beta, mn, og) : mn;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    const int64_t gr = r0 + r;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    if (gr < P.hr) {
      const int64_t base = (P.row0 + gr) * P.cols;
      if (vec_rows && c + 3 < P.cols) {
        float g[4], m[4], mn[4];
        load4<GBF16>(P.grad, base + c, g);
        load4<false>(P.mom, base + c, m);
#pragma unroll
        for (int e = 0; e < 4; ++e) one(g[e], m[e], mn[e], u[e]);
        store4(P.mom, base + c, mn, false);
        store4(orig, gr * P.orig_ld + c, u, xb);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + e < P.cols) {
            float mn;
            one(load_as_f32<GBF16>(P.grad, base + c + e), P.mom[base + c + e], mn, u[e]);
            P.mom[base + c + e] = mn;
            if (xb) store_from_f32<true>(orig, gr * P.orig_ld + c + e, u[e]);
            else store_from_f32<false>(orig, gr * P.orig_ld + c + e, u[e]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(u[e], u[e], ss);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[r][cq + e] = u[e];
  }
  __syncthreads();
  // transposed copy: row (c0 + cc) of the transposed block, elements r0 + 4 rq .. + 3
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = threadIdx.x + 256 * k;
    const int cc = q >> 4, rq = (q & 15) * 4;
    const int64_t gc = c0 + cc, gr = r0 + rq;
    if (gc >= P.cols || gr >= P.hr) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = tile[rq + e][cc];
    if (gr + 3 < P.hr) {
      store4(trans, gc * P.trans_ld + gr, v, xb);
    } else {
      for (int e = 0; e < 4 && gr + e < P.hr; ++e) {
        if (xb) store_from_f32<true>(trans, gc * P.trans_ld + gr + e, v[e]);
        else store_from_f32<false>(trans, gc * P.trans_ld + gr + e, v[e]);
      }
    }
  }
  // block sum of squares: wave butterfly, then the 4 waves in order
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) partials[t] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ----------------------------------------------------------------- KN

__global__ __launch_bounds__(256) void kn_finalize(const K1Prob *probs, const float *partials, float *scales,
                                                   float eps, const int32_t *skip) {
  if (skip && *skip) return;
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

// One IEEE multiply per element.  8 elements per lane when the chunk's
// source and destination are 16-byte aligned.  Returns this thread's sum of
// squares of the values it wrote, in its own element order.
template <bool SBF16>
__device__ __forceinline__ float k3_body(const K3Run &R, int64_t start, int64_t end) {
  const void *src = R.src;
  float ss = 0.f;
  const bool vec = aligned16(R.dst + start) &&
                   aligned16(SBF16 ? (const void *)(static_cast<const uint16_t *>(src) + R.first + start)
                                   : (const void *)(static_cast<const float *>(src) + R.first + start));
  if (vec && end - start == K3_CHUNK) {
    // a whole chunk: two 8-element groups per lane, both loads first
    const int64_t j0 = start + 8 * threadIdx.x, j1 = j0 + 8 * 256;
    float v0[8], v1[8];
    load8<SBF16>(src, R.first + j0, v0);
    load8<SBF16>(src, R.first + j1, v1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v0[k] = v0[k] * R.scale;
      ss = fmaf(v0[k], v0[k], ss);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v1[k] = v1[k] * R.scale;
      ss = fmaf(v1[k], v1[k], ss);
    }
    store8_f32(R.dst + j0, v0);
    store8_f32(R.dst + j1, v1);
    return ss;
  }
  if (vec) {
    int64_t j;
    for (j = start + 8 * threadIdx.x; j + 8 <= end; j += 8 * 256) {
      float v[8];
      load8<SBF16>(src, R.first + j, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[k] = v[k] * R.scale;
        ss = fmaf(v[k], v[k], ss);
      }
      store8_f32(R.dst + j, v);
    }
    for (j = start + (end - start) / 8 * 8 + threadIdx.x; j < end; j += 256) {
      const float v = load_as_f32<SBF16>(src, R.first + j) * R.scale;
      R.dst[j] = v;
      ss = fmaf(v, v, ss);
    }
    return ss;
  }
  for (int64_t j = start + threadIdx.x; j < end; j += 256) {
    const float v = load_as_f32<SBF16>(src, R.first + j) * R.scale;
    R.dst[j] = v;
    ss = fmaf(v, v, ss);
  }
  return ss;
}

// Workgroup sum of one value per thread in a fixed order: wave butterfly,
// then the four waves in index order.  Result valid in thread 0.
__device__ __forceinline__ float block_sum_fixed(float v) {
  __shared__ float red[4];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k3_scatter(const K3Run *runs, int nrun, const int32_t *skip, float *nparts,
                                                  int64_t pbase) {
  if (skip && *skip) return;
  const int64_t ch = blockIdx.x;
  const int i = find_owner(nrun, ch, [&](int k) { return runs[k].chunk0; });
  const K3Run R = runs[i];
  const int64_t start = (ch - R.chunk0) * K3_CHUNK;
  const int64_t end = min(start + (int64_t)K3_CHUNK, R.length);
  const float ss = R.src_bf16 ? k3_body<true>(R, start, end) : k3_body<false>(R, start, end);
  if (nparts) {
    const float t = block_sum_fixed(ss);
    if (threadIdx.x == 0) nparts[pbase + ch] = t;
  }
}

// ----------------------------------------------------------------- finite check

__global__ __launch_bounds__(64) void kf_zero(int32_t *flag) {
  if (threadIdx.x == 0) *flag = 0;
}

template <bool GBF16>
__global__ __launch_bounds__(256) void kf_scan(const K0Mat *mats, int nmat, int32_t *flag) {
  const int64_t ch = blockIdx.x;
  const int i = find_owner(nmat, ch, [&](int k) { return mats[k].chunk0; });
  const void *g = mats[i].g;
  const int64_t start = (ch - mats[i].chunk0) * K0_CHUNK;
  const int64_t end = min(start + (int64_t)K0_CHUNK, mats[i].numel);
  int bad = 0;
  for (int64_t j = start + threadIdx.x; j < end; j += 256) {
    const float v = load_as_f32<GBF16>(g, j);
    bad |= !isfinite(v);
  }
  // every writer stores the same value 1, so concurrent stores agree
  if (__syncthreads_or(bad) && threadIdx.x == 0) *flag = 1;
}

// ----------------------------------------------------------------- norm, clip, apply

// Two-level fixed-order sum of the writeback's chunk partials: level 1 sums
// kNormSpan consecutive partials per workgroup, level 2 (one workgroup)
// sums the level-1 results, both in fp64 with a fixed thread / tree order.

__device__ __forceinline__ double block_sum_f64(double s) {
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(256) void k_norm_level1(const float *nparts, int64_t n, double *l1,
                                                     const int32_t *skip) {
  if (skip && *skip) return;
  const int64_t b = (int64_t)blockIdx.x * kNormSpan;
  const int64_t e = min(b + (int64_t)kNormSpan, n);
  double s = 0.0;
  for (int64_t i = b + threadIdx.x; i < e; i += 256) s += (double)nparts[i];
  const double t = block_sum_f64(s);
  if (threadIdx.x == 0) l1[blockIdx.x] = t;
}

__global__ __launch_bounds__(256) void k_norm_clip(const double *l1, int n1, float max_norm, float *nc,
                                                   float *user_out, const int32_t *skip) {
  if (skip && *skip) return;
  double s = 0.0;
  for (int i = threadIdx.x; i < n1; i += 256) s += l1[i];
  const double tot = block_sum_f64(s);
  if (threadIdx.x == 0) {
    const double norm = sqrt(tot);
    double clip = 1.0;
    if (max_norm > 0.f) clip = fmin(1.0, (double)max_norm / (norm + 1e-6));
    nc[0] = (float)norm;
    nc[1] = (float)clip;
    if (user_out) {
      user_out[0] = (float)norm;
      user_out[1] = (float)clip;
    }
  }
}

__global__ __launch_bounds__(256) void k_apply(const KARun *runs, int nrun, const float *nc, float lr, float wd,
                                               const int32_t *skip) {
  if (skip && *skip) return;
  const int64_t ch = blockIdx.x;
  const int i = find_owner(nrun, ch, [&](int k) { return runs[k].chunk0; });
  const KARun R = runs[i];
  const int64_t start = (ch - R.chunk0) * KA_CHUNK;
  const int64_t end = min(start + (int64_t)KA_CHUNK, R.length);
  const float decay = 1.0f - lr * wd;
  const float step = lr * nc[1];
  auto one = [&](float p, float u) { return fmaf(-step, u, p * decay); };
  if (aligned16(R.param + start) && aligned16(R.upd + start) && end - start == KA_CHUNK) {
    const int64_t j0 = start + 8 * threadIdx.x, j1 = j0 + 8 * 256;
    float p0[8], u0[8], p1[8], u1[8];
    load8<false>(R.param, j0, p0);
    load8<false>(R.upd, j0, u0);
    load8<false>(R.param, j1, p1);
    load8<false>(R.upd, j1, u1);
#pragma unroll
    for (int k = 0; k < 8; ++k) { p0[k] = one(p0[k], u0[k]); p1[k] = one(p1[k], u1[k]); }
    store8_f32(R.param + j0, p0);
    store8_f32(R.param + j1, p1);
    return;
  }
  if (aligned16(R.param + start) && aligned16(R.upd + start)) {
    int64_t j;
    for (j = start + 8 * threadIdx.x; j + 8 <= end; j += 8 * 256) {
      float p[8], u[8];
      load8<false>(R.param, j, p);
      load8<false>(R.upd, j, u);
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] = one(p[k], u[k]);
      store8_f32(R.param + j, p);
    }
    for (j = start + (end - start) / 8 * 8 + threadIdx.x; j < end; j += 256) R.param[j] = one(R.param[j], R.upd[j]);
    return;
  }
  for (int64_t j = start + threadIdx.x; j < end; j += 256) R.param[j] = one(R.param[j], R.upd[j]);
}

// ----------------------------------------------------------------- KC

__global__ __launch_bounds__(256) void kc_copy_scaled(const ProbDev *probs, const K1Prob *k1, char *ws,
                                                      const float *scales, const int32_t *skip) {
  if (skip && *skip) return;
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
                     float grad_scale, const int32_t *skip, bool gbf16, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  const float omb = 1.0f - beta;
  dim3 g((unsigned)tiles), b(256);
  if (gbf16)
    hipLaunchKernelGGL(k1_momentum<true>, g, b, 0, s, probs, nprob, ws, partials, beta, omb, nesterov, grad_scale, skip);
  else
    hipLaunchKernelGGL(k1_momentum<false>, g, b, 0, s, probs, nprob, ws, partials, beta, omb, nesterov, grad_scale, skip);
  return hipGetLastError();
}

hipError_t launch_kn(const K1Prob *probs, int nprob, const float *partials, float *scales, float eps,
                     const int32_t *skip, hipStream_t s) {
  if (nprob <= 0) return hipSuccess;
  hipLaunchKernelGGL(kn_finalize, dim3(nprob), dim3(256), 0, s, probs, partials, scales, eps, skip);
  return hipGetLastError();
}

hipError_t launch_k3(const K3Run *runs, int nrun, int64_t chunks, const int32_t *skip, float *nparts, int64_t pbase,
                     hipStream_t s) {
  if (chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k3_scatter, dim3((unsigned)chunks), dim3(256), 0, s, runs, nrun, skip, nparts, pbase);
  return hipGetLastError();
}

hipError_t launch_kc(const ProbDev *probs, const K1Prob *k1, int nprob, char *ws, const float *scales,
                     const int32_t *skip, hipStream_t s) {
  if (nprob <= 0) return hipSuccess;
  hipLaunchKernelGGL(kc_copy_scaled, dim3(nprob), dim3(256), 0, s, probs, k1, ws, scales, skip);
  return hipGetLastError();
}

hipError_t launch_finite(const K0Mat *mats, int nmat, int64_t chunks, bool gbf16, int32_t *flag, hipStream_t s) {
  hipLaunchKernelGGL(kf_zero, dim3(1), dim3(64), 0, s, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks <= 0) return e;
  if (gbf16) hipLaunchKernelGGL(kf_scan<true>, dim3((unsigned)chunks), dim3(256), 0, s, mats, nmat, flag);
  else hipLaunchKernelGGL(kf_scan<false>, dim3((unsigned)chunks), dim3(256), 0, s, mats, nmat, flag);
  return hipGetLastError();
}

hipError_t launch_norm_clip(const float *nparts, int64_t n, double *l1, float max_norm, float *nc, float *user_out,
                            const int32_t *skip, hipStream_t s) {
  const int n1 = (int)((n + kNormSpan - 1) / kNormSpan);
  if (n1 > 0) {
    hipLaunchKernelGGL(k_norm_level1, dim3((unsigned)n1), dim3(256), 0, s, nparts, n, l1, skip);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_norm_clip, dim3(1), dim3(256), 0, s, l1, n1, max_norm, nc, user_out, skip);
  return hipGetLastError();
}

hipError_t launch_apply(const KARun *runs, int nrun, int64_t chunks, const float *nc, float lr, float wd,
                        const int32_t *skip, hipStream_t s) {
  if (chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_apply, dim3((unsigned)chunks), dim3(256), 0, s, runs, nrun, nc, lr, wd, skip);
  return hipGetLastError();
}

}  // namespace muon
