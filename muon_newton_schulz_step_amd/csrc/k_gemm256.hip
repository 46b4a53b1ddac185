// Large-tile grouped Newton-Schulz GEMM for bf16 operands on gfx950.
//
// Same contract as ns_gemm (C = s^p (cd D + cacc A B^T) + cdiag I over a
// tile list, both operands row-major with K contiguous), for problems whose
// small side is at least 256:
//  - 256 x 256 output tile per workgroup of 4 wave64s (2 x 2), each wave
//    128 x 128 = 8 x 8 blocks of v_mfma_f32_16x16x32_bf16, 256 fp32
//    accumulators per lane.  Per 32-deep K step a wave reads 16 KB of
//    operands from LDS for 64 MFMAs.  The 16 x 16 x 32 form issues the same
//    flops as 32 x 32 x 16 in half-length instructions and, measured on this
//    kernel, runs the whole step 5% faster (the register-only issue rate of
//    the two differs by 11%, partly through the clock the chip holds); its
//    accumulation order gives bitwise the same results here.
//  - K staged 64 deep (128-byte rows) straight from global memory into LDS
//    with 16-byte LDS-DMA loads (buffer_load_dwordx4 ... lds: lane L lands
//    at base + 16 L), double buffered.  A stage is two k-steps with two
//    barriers: one in the first k-step once every wave has read the stage's
//    fragments, which frees its buffer for the DMA of stage t+2 (spread one
//    instruction per group of four MFMAs over the rest of the stage), one
//    between the k-steps that waits for stage t+1 only.  Issued back to back
//    the DMA instructions stall the wave (and its MFMAs) until the address
//    unit drains them.  A ragged last stage (K not a multiple of 64) goes
//    through registers so elements at k >= K are zeroed.
//  - 16-byte chunks of each row are XOR-swizzled (position = chunk ^ f(row))
//    so the 16 rows each quarter of a fragment read touches spread over all
//    LDS banks.
//  - Workgroup i runs on XCD i mod 8; the tile list (ordered in 4 x 8
//    blocks per problem) is cut into chunks of 256 and XCD x takes entries
//    [32 x, 32 x + 32) of each chunk, so the 32 CUs of an XCD work on one
//    block and share its operand panels in their L2 (measured L2 hit rate
//    of the stage loads is otherwise about 50%).
//  - A split product (hi.hi + hi.lo + lo.hi of bf16 hi/lo pairs) runs its
//    three K segments back to back through the same pipeline and
//    accumulators: stage kt of the concatenated range reads segment
//    kt / nk, whose operands sit at fixed byte offsets from segment 0's.
// Rows beyond M or N are clamped to the last valid row when loading; they
// only feed outputs that are never stored.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "elem.hpp"
#include "tables.hpp"

#ifndef MUON_LDS_SWIZZLE
#define MUON_LDS_SWIZZLE 1
#endif
#ifndef MUON_XCD_REMAP
#define MUON_XCD_REMAP 1
#endif

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int BT = 256;            // output tile edge
constexpr int KS = 64;             // K elements per stage
constexpr int ROWB = 128;          // bytes per staged row (64 bf16)
constexpr int OPB = BT * ROWB;     // 32 KB per operand per stage
constexpr int NTHR = 256;
constexpr int NXCD = 8;
constexpr int XCD_CUS = 32;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r, int c) {
#if MUON_LDS_SWIZZLE == 0
  return c ^ (r & 7);
#else
  return c ^ ((r >> 1) & 7);
#endif
}

// c += a b on v_mfma_f32_16x16x32_bf16.  In the main loop the accumulator
// is tied in place through inline asm (the compiler's own selection of the
// instruction picks a destination apart from the accumulator and rotates 64
// blocks through copies every loop trip); the compiler does not see the
// latency of those, so every accumulator's last product (the tile's final
// k-step, LAST) goes through the builtin, whose result latency the compiler
// covers before anything reads it.  An asm product is then read only by the
// MFMAs of the next k-step, 64 instructions later.
template <bool LAST = false>
__device__ __forceinline__ void mfma16(f32x4_t &c, const bf16x8_t &a, const bf16x8_t &b) {
  if constexpr (LAST) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)pk2(f, 0.f); }

__device__ __forceinline__ void store_elem(char *base, int64_t idx, float v, bool f32) {
  if (f32) reinterpret_cast<float *>(base)[idx] = v;
  else reinterpret_cast<uint16_t *>(base)[idx] = f2bf(v);
}

__device__ __forceinline__ float load_elem(const char *base, int64_t idx, bool f32) {
  return f32 ? reinterpret_cast<const float *>(base)[idx] : bf2f(reinterpret_cast<const uint16_t *>(base)[idx]);
}

// Store n (<= 8) consecutive values at element index idx: one 16-byte
// (bf16) or two 16-byte (fp32) stores when the chunk is whole and aligned,
// element stores otherwise.
__device__ __forceinline__ void store_chunk(char *base, int64_t idx, const float *v, int n, bool f32) {
  if (f32) {
    float *p = reinterpret_cast<float *>(base) + idx;
    if (n == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      for (int e = 0; e < n; ++e) p[e] = v[e];
    }
  } else {
    uint16_t *p = reinterpret_cast<uint16_t *>(base) + idx;
    if (n == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      uint4 w;
      w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      w.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
      w.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
      *reinterpret_cast<uint4 *>(p) = w;
    } else {
      for (int e = 0; e < n; ++e) p[e] = f2bf(v[e]);
    }
  }
}

// Store / load n (<= 4) consecutive values: one vector access (8 bytes
// bf16, 16 bytes fp32) when the quad is whole and aligned, elements otherwise.
__device__ __forceinline__ void store_quad(char *base, int64_t idx, const float *v, int n, bool f32) {
  if (f32) {
    float *p = reinterpret_cast<float *>(base) + idx;
    if (n == 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else for (int e = 0; e < n; ++e) p[e] = v[e];
  } else {
    uint16_t *p = reinterpret_cast<uint16_t *>(base) + idx;
    if (n == 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      uint2 w;
      w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      *reinterpret_cast<uint2 *>(p) = w;
    } else {
      for (int e = 0; e < n; ++e) p[e] = f2bf(v[e]);
    }
  }
}

__device__ __forceinline__ void load_quad(const char *base, int64_t idx, float *v, int n, bool f32) {
  if (f32) {
    const float *p = reinterpret_cast<const float *>(base) + idx;
    if (n == 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      const float4 w = *reinterpret_cast<const float4 *>(p);
      v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    } else {
      for (int e = 0; e < n; ++e) v[e] = p[e];
    }
  } else {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + idx;
    if (n == 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      const uint2 w = *reinterpret_cast<const uint2 *>(p);
      v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
      v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      for (int e = 0; e < n; ++e) v[e] = bf2f(p[e]);
    }
  }
}

// 8 bf16 <-> floats, 16-byte aligned
__device__ __forceinline__ void unpack8(const uint4 w, float *v) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    v[2 * d] = __uint_as_float(a[d] << 16);
    v[2 * d + 1] = __uint_as_float(a[d] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float *v) {
  return make_uint4(pk2(v[0], v[1]), pk2(v[2], v[3]), pk2(v[4], v[5]), pk2(v[6], v[7]));
}

// 16-byte nontemporal store (the outputs are read back by the next launch,
// long after they would have left the L2)
__device__ __forceinline__ void st16(char *p, uint4 v) {
  __builtin_nontemporal_store(v.x, reinterpret_cast<uint32_t *>(p));
  __builtin_nontemporal_store(v.y, reinterpret_cast<uint32_t *>(p) + 1);
  __builtin_nontemporal_store(v.z, reinterpret_cast<uint32_t *>(p) + 2);
  __builtin_nontemporal_store(v.w, reinterpret_cast<uint32_t *>(p) + 3);
}

// hi = the bf16 value nearest v, lo = v - hi (then rounded to bf16 when
// stored): hi + lo carries about 16 significant bits of v
__device__ __forceinline__ void split4(const float *v, float *hi, float *lo) {
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    const uint32_t h = pk2(v[e], v[e + 1]);
    hi[e] = __uint_as_float(h << 16);
    hi[e + 1] = __uint_as_float(h & 0xffff0000u);
    lo[e] = v[e] - hi[e];
    lo[e + 1] = v[e + 1] - hi[e + 1];
  }
}

__device__ __forceinline__ uint4 mask_tail_bf16(uint4 v, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t keep = (2 * d < valid ? 0x0000ffffu : 0u) | (2 * d + 1 < valid ? 0xffff0000u : 0u);
    w[d] &= keep;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Source of one stage of the concatenated K range: the operand bases of its
// segment and the K offset inside that segment.
struct Src {
  const char *a, *b;
  int64_t k0;
};

// SPLIT: the recipe may carry K segments, a split D and a split output; the
// plain instance keeps the single-segment pipeline free of them.
// LDS of both kernels: two stage buffers of both operands (the epilogue
// stages through the first 66 KB), then a slot through which the
// persistent kernel hands a work item to every wave.
constexpr int LDS_SLOT = 2 * 2 * OPB;
__shared__ __attribute__((aligned(1024))) char lds[LDS_SLOT + 64];

// One 256 x 256 output tile of recipe R: main loop and epilogue.  tid is
// the thread's index in the workgroup.
template <bool SPLIT>
__device__ __forceinline__ void gemm_tile(const ProbDev *probs, char *ws, const float *scales, const GemmRecipe R,
                                          const TileDev tile, const int tid) {
  const ProbDev &P = probs[tile.prob];
  const int64_t M = R.dimM ? P.n : P.m;
  const int64_t N = R.dimN ? P.n : P.m;
  const int64_t K = R.dimK ? P.n : P.m;
  const char *A = ws + P.off[R.rA];
  const char *B = ws + P.off[R.rB];
  const int64_t lda = P.ld[R.rA], ldb = P.ld[R.rB];
  // K segments 1, 2 of a split product read (rA2[s-1], rB2[s-1]), which the
  // planner lays out with the leading dimensions of rA and rB
  int64_t dA1 = 0, dA2 = 0, dB1 = 0, dB2 = 0;
  if (SPLIT && R.nseg > 1) {
    dA1 = P.off[R.rA2[0]] - P.off[R.rA]; dB1 = P.off[R.rB2[0]] - P.off[R.rB];
  }
  if (SPLIT && R.nseg > 2) {
    dA2 = P.off[R.rA2[1]] - P.off[R.rA]; dB2 = P.off[R.rB2[1]] - P.off[R.rB];
  }
  const int64_t m0 = (int64_t)tile.tm * BT, n0 = (int64_t)tile.tn * BT;

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lg = lane >> 4;

  // loader geometry: wave w stages rows [64 w, 64 w + 64) of both operands,
  // 8 rows (1 KB) per instruction; lane L covers row 64w + 8j + L/8, LDS
  // chunk position L%8, which holds global chunk swz(row, L%8).
  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

  const int lrow = lane >> 3, lpos = lane & 7;
  int64_t arow[8], brow[8];
  int lchunk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + lrow;
    arow[j] = min(m0 + r, M - 1) * lda;
    brow[j] = min(n0 + r, N - 1) * ldb;
    lchunk[j] = swz(r, lpos) * 8;
  }
  // Whole stages load as buffer loads into LDS: a descriptor per operand
  // panel (scalar registers, based at the tile's first row and the stage's K
  // offset) and a 32-bit byte offset per lane, instead of a 64-bit address
  // per lane and instruction.
  auto uni = [](const char *ptr) {
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
  };
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    aoff[j] = (uint32_t)((arow[j] - m0 * lda + lchunk[j]) * 2);
    boff[j] = (uint32_t)((brow[j] - n0 * ldb + lchunk[j]) * 2);
  }
  const int nfull = (int)(K / KS);
  const int nk = (int)((K + KS - 1) / KS);
  const int nkt = SPLIT ? nk * R.nseg : nk;          // stages over all K segments

  // stage kt of the concatenated range into LDS buffer st: full stages by
  // LDS-DMA, a ragged one through registers with k >= K zeroed
  auto stage = [&](int kt, int st) {
    const int seg = !SPLIT ? 0 : (kt >= nk ? (kt >= 2 * nk ? 2 : 1) : 0);
    const int kk = kt - seg * nk;
    const char *a = A + (seg == 0 ? 0 : (seg == 1 ? dA1 : dA2));
    const char *b = B + (seg == 0 ? 0 : (seg == 1 ? dB1 : dB2));
    const int64_t k0 = (int64_t)kk * KS;
    char *la = lds + st * 2 * OPB;
    char *lb = la + OPB;
    if (kk < nfull) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (wave * 64 + j * 8) * ROWB;
        __builtin_amdgcn_global_load_lds(a + (arow[j] + k0 + lchunk[j]) * 2, (lds_void *)(la + off), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(b + (brow[j] + k0 + lchunk[j]) * 2, (lds_void *)(lb + off), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t gk = k0 + lchunk[j];
        const int valid = (int)min<int64_t>(K - gk, 8);
        uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
        if (valid > 0) {
          va = *reinterpret_cast<const uint4 *>(a + (arow[j] + gk) * 2);
          vb = *reinterpret_cast<const uint4 *>(b + (brow[j] + gk) * 2);
          if (valid < 8) { va = mask_tail_bf16(va, valid); vb = mask_tail_bf16(vb, valid); }
        }
        const int off = (wave * 64 + j * 8) * ROWB + lane * 16;
        *reinterpret_cast<uint4 *>(la + off) = va;
        *reinterpret_cast<uint4 *>(lb + off) = vb;
      }
    }
  };

  // Fragments of v_mfma_f32_16x16x32_bf16 over a 32-deep k-step: lane L of
  // block i holds row 16 i + L%16 of the wave's 128 rows, K elements
  // 8 (L/16) .. +8 of the step, i.e. 16-byte chunk 4 ks + L/16 of the staged
  // row.  Block rows are 16 apart, so a lane's swizzle key is the same for
  // all eight blocks, and the second step's chunks are the first step's with
  // bit 2 flipped: one LDS address per lane and operand, the block and step
  // folded into immediate offsets.
  const int pos0 = swz(lr, lg) * 16;
  const int abase = (wm * 128 + lr) * ROWB + pos0;
  const int bbase = (wn * 128 + lr) * ROWB + pos0;
  bf16x8_t fa[2][8], fb[2][8];
  auto rdA = [&](int set, int st, int ks, int i) {
    const char *la = lds + st * 2 * OPB;
    fa[set][i] = *reinterpret_cast<const bf16x8_t *>(la + ((abase + i * 16 * ROWB) ^ (ks * 64)));
  };
  auto rdB = [&](int set, int st, int ks, int j) {
    const char *lb = lds + st * 2 * OPB + OPB;
    fb[set][j] = *reinterpret_cast<const bf16x8_t *>(lb + ((bbase + j * 16 * ROWB) ^ (ks * 64)));
  };
  auto read_frags = [&](int set, int st, int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) rdA(set, st, ks, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) rdB(set, st, ks, j);
  };
  // read q of a k-step in the order the MFMAs consume them: A0, B0..B7, A1..A7
  auto read1 = [&](int set, int st, int ks, int q) {
    if (q == 0) rdA(set, st, ks, 0);
    else if (q <= 8) rdB(set, st, ks, q - 1);
    else rdA(set, st, ks, q - 8);
  };
  // One 32-deep k-step on fragment set `set` (the ragged-K pipeline): 16
  // groups of four MFMAs (one block row, four block columns) with the 16
  // fragment reads of the next step (stage buffer rst, k-step rks) in
  // groups 0..11, two in each of groups 0..3, so they land four groups
  // before the next step needs them.  sched_barrier keeps this order.
  auto kstep = [&](int set, int rst, int rks, auto last) {
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int i = n >> 1, j = (n & 1) * 4;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) mfma16<decltype(last)::value>(acc[i][j + jj], fa[set][i], fb[set][j + jj]);
      __builtin_amdgcn_sched_barrier(0);
      if (n < 4) { read1(set ^ 1, rst, rks, 2 * n); read1(set ^ 1, rst, rks, 2 * n + 1); }
      else if (n < 12) read1(set ^ 1, rst, rks, n + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (nfull == nk) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto src_of = [&](int kt) {
      Src r{A, B, (int64_t)kt * KS};
      if (SPLIT) {
        const bool s1 = kt >= nk, s2 = kt >= 2 * nk;
        r.a = A + (s2 ? dA2 : (s1 ? dA1 : 0));
        r.b = B + (s2 ? dB2 : (s1 ? dB1 : 0));
        r.k0 = (int64_t)(kt - (s2 ? 2 * nk : (s1 ? nk : 0))) * KS;
      }
      return r;
    };
    // descriptor word 3 of a raw dword buffer on gfx9 (32-bit data format)
    constexpr int kRsrcWord3 = 0x00020000;
    auto dma1 = [&](const Src &sr, int st, int q) {
      char *la = lds + st * 2 * OPB + wv * 64 * ROWB;
      const int j = q & 7;
      if (q < 8) {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)uni(sr.a + (m0 * lda + sr.k0) * 2), (short)0,
                                                          0x7fffffff, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(la + j * 8 * ROWB), 16, aoff[j], 0, 0, 0);
      } else {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)uni(sr.b + (n0 * ldb + sr.k0) * 2), (short)0,
                                                          0x7fffffff, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(la + OPB + j * 8 * ROWB), 16, boff[j], 0, 0, 0);
      }
    };
    {
      const Src s0 = src_of(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) dma1(s0, 0, q);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nkt > 1) {
      const Src s1 = src_of(1);
#pragma unroll
      for (int q = 0; q < 16; ++q) dma1(s1, 1, q);
    }
    read_frags(0, 0, 0);
    // One stage, two barriers.  k-step 0 reads k-step 1's fragments in its
    // groups 0..7 (two per group); barrier 1 after group 9 (every wave done
    // reading this stage's buffer) frees the buffer, and stage kt+2's 16 DMA
    // instructions follow: one per group over groups 10..15 of k-step 0,
    // then ten spread over the 16 groups of k-step 1.  Barrier 2 at the end
    // of k-step 0 waits for stage kt+1 only (every load but the six issued
    // since), so k-step 1 can read it.  Spreading the stage's loads over 22
    // groups instead of one k-step measured 3.5-4.3% faster: the address
    // unit takes them as they come instead of stalling the wave's MFMAs.
    // The last two stages are peeled off with those loads compiled out.
    constexpr int kBar1 = 9;                // group of k-step 0 ending with barrier 1
    constexpr int kDma0 = 15 - kBar1;       // DMA instructions in k-step 0
    constexpr int kDma1 = 16 - kDma0;       // in k-step 1
    static_assert(kDma0 == 6, "the vmcnt immediate of barrier 2");
    auto body = [&](int kt, auto load, auto last) {
      constexpr bool LOAD = decltype(load)::value;
      constexpr bool LAST = decltype(last)::value;
      const int st = kt & 1;
      const Src nn = src_of(LOAD ? kt + 2 : kt);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int i = n >> 1, j = (n & 1) * 4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) mfma16(acc[i][j + jj], fa[0][i], fb[0][j + jj]);
        __builtin_amdgcn_sched_barrier(0);
        if (n < 8) { read1(1, st, 1, 2 * n); read1(1, st, 1, 2 * n + 1); }
        if (n == kBar1) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if constexpr (LOAD) {
          if (n > kBar1) dma1(nn, st, n - kBar1 - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (LOAD) asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int i = n >> 1, j = (n & 1) * 4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) mfma16<LAST>(acc[i][j + jj], fa[1][i], fb[1][j + jj]);
        __builtin_amdgcn_sched_barrier(0);
        if (n < 4) { read1(0, st ^ 1, 0, 2 * n); read1(0, st ^ 1, 0, 2 * n + 1); }
        else if (n < 12) read1(0, st ^ 1, 0, n + 4);
        if constexpr (LOAD) {
          // the q-th of the last kDma1 instructions in the group where
          // n kDma1 / 16 steps up
          if (((n + 1) * kDma1) / 16 > (n * kDma1) / 16) dma1(nn, st, kDma0 + (n * kDma1) / 16);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    int kt = 0;
    for (; kt < nkt - 2; ++kt) body(kt, yes, no);
    if (kt == nkt - 2) { body(kt, no, no); ++kt; }
    body(kt, no, yes);
  } else {
    // K not a multiple of 64: the same pipeline, stages loaded by stage()
    stage(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nkt > 1) stage(1, 1);
    read_frags(0, 0, 0);
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    auto rstage = [&](int kt, auto last) {
      const int st = kt & 1;
      kstep(0, st, 1, no);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 2 < nkt) stage(kt + 2, st);
      kstep(1, st ^ 1, 0, last);
    };
    for (int kt = 0; kt < nkt - 1; ++kt) rstage(kt, no);
    rstage(nkt - 1, yes);
  }

  // ---- epilogue: C = s^p (cd D + cacc acc) + cdiag I, stored to S0/S1.
  // The tile leaves registers in four passes of 64 rows (block row p of
  // both wave rows), staged as fp32 in LDS with row stride 264 floats (the
  // two half-waves of an accumulator write land in opposite bank halves):
  //   phase 1: accumulators -> LDS (times cacc)
  //   phase 2: 4-float row quads (a wave touches 1 KB contiguous): + cd D
  //            (vector reads of D), scale, diagonal; final values back to
  //            LDS; row-major stores.  Runs even when every output is
  //            transposed, since it produces the final values.
  //   phase 3: 8-row column chunks -> transposed stores and the mirror tile
  //            of symmetric outputs (16 bytes per lane for bf16)
  __syncthreads();
  float *stg = reinterpret_cast<float *>(lds);
  constexpr int SLD = 264;  // staging row stride (floats)
  float sc = 1.f;
  if (R.scale_pow) {
    const float sv = scales[tile.prob];
    sc = R.scale_pow == 2 ? sv * sv : sv;
  }
  const bool mirror = (R.flags & GF_SYM) && tile.tm != tile.tn;
  const bool t0 = (R.flags & GF_S0_TRANS) || ((R.flags & GF_S0_PROBT) && (P.flags & PF_TALL));
  const bool t1 = (R.flags & GF_S1_TRANS) != 0;
  const bool f0 = (R.flags & GF_S0_F32) != 0, f1 = (R.flags & GF_S1_F32) != 0, fd = (R.flags & GF_D_F32) != 0;
  const bool diag = (R.flags & GF_DIAG) != 0;
  const char *D = R.rD >= 0 ? ws + P.off[R.rD] : nullptr;
  const int64_t ldd = R.rD >= 0 ? P.ld[R.rD] : 0;
  const bool dsplit = SPLIT && (R.flags & GF_D_SPLIT) != 0;
  const char *D2 = dsplit ? ws + P.off[R.rD2] : nullptr;
  const bool osplit = SPLIT && (R.flags & GF_SPLIT_OUT) != 0;
  char *S0 = ws + P.off[R.rS0];
  const int64_t ld0 = P.ld[R.rS0];
  char *S1 = R.rS1 >= 0 ? ws + P.off[R.rS1] : nullptr;
  const int64_t ld1 = R.rS1 >= 0 ? P.ld[R.rS1] : 0;
  const bool col_phase = t0 || (S1 && t1) || mirror;
  // the scale is folded into the staged accumulators, so staged values are
  // final unless D or the diagonal change them: only then does the row
  // phase write its values back for the column phase
  const float cs = R.cacc * sc, cds = R.cd * sc;
  const bool wback = col_phase && (D != nullptr || diag);
  // Interior tile with bf16 operands and 16-byte aligned rows: the row phase
  // takes 8-column chunks with the D chunks of a pass loaded up front, so no
  // wait on the vector-memory counter (which also counts stores) falls
  // between its stores.
  const bool fast = m0 + BT <= M && n0 + BT <= N && !f0 && !f1 && !fd && (ld0 & 7) == 0 &&
                    (!S1 || (ld1 & 7) == 0) && (!D || (ldd & 7) == 0);

  // Staged row r (0..63) = 8-row group g = r / 8, element e = r % 8 lives in
  // LDS row 8 g + (e + 2 (g % 4)) % 8: the column gather of the transposed
  // stores (rows 8 k + e of one column for k = 0..3 across lanes) then hits
  // 64 distinct banks, and the two half-waves of an accumulator write still
  // land 32 banks apart.
  auto srow = [](int r) { return (r & ~7) | ((r + ((r >> 3) & 3) * 2) & 7); };
  // block (i, j) of 16 x 16: lane L holds rows 4 (L/16) .. +4, column L%16
  auto put = [&](const f32x4_t &blk, int ih, int j) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * 32 + ih * 16 + 4 * lg + v;
      stg[srow(r) * SLD + wn * 128 + j * 16 + lr] = blk[v] * cs;
    }
  };
#pragma unroll 1
  for (int p = 0; p < 4; ++p) {
    if (p) __syncthreads();
    // staging row r (0..63) is tile row (r / 32) * 128 + p * 32 + r % 32;
    // fast row phase: chunk q of thread tid is row (tid + 256 q) / 32,
    // columns 8 ((tid + 256 q) % 32) .. +8
    uint4 dq[8], dq2[8];
    if (fast && D) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int ch = tid + NTHR * q;
        const int r = ch >> 5, c8 = (ch & 31) * 8;
        const int64_t gi = m0 + (r >> 5) * 128 + p * 32 + (r & 31);
        const int64_t e = gi * ldd + n0 + c8;
        dq[q] = *reinterpret_cast<const uint4 *>(D + e * 2);
        if (dsplit) dq2[q] = *reinterpret_cast<const uint4 *>(D2 + e * 2);
      }
    }
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      if (p == pp) {
#pragma unroll
        for (int ih = 0; ih < 2; ++ih)
#pragma unroll
          for (int j = 0; j < 8; ++j) put(acc[2 * pp + ih][j], ih, j);
      }
    }
    __syncthreads();
    // fast row phase; HAS_D: D chunks in dq (and dq2 when split)
    auto row_fast = [&](auto has_d) {
      constexpr bool HAS_D = decltype(has_d)::value;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int ch = tid + NTHR * q;
        const int r = ch >> 5, c8 = (ch & 31) * 8;
        const int64_t gi = m0 + (r >> 5) * 128 + p * 32 + (r & 31);
        const int64_t gj = n0 + c8;
        float *src = stg + srow(r) * SLD + c8;
        const float4 a4 = *reinterpret_cast<const float4 *>(src);
        const float4 b4 = *reinterpret_cast<const float4 *>(src + 4);
        float v[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
        if constexpr (HAS_D) {
          float dv[8];
          unpack8(dq[q], dv);
          if (dsplit) {
            float dl[8];
            unpack8(dq2[q], dl);
#pragma unroll
            for (int e = 0; e < 8; ++e) dv[e] += dl[e];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = fmaf(cds, dv[e], v[e]);
        }
        if (diag) {
          const int64_t dd = gi - gj;
          if (dd >= 0 && dd < 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e == dd) v[e] += R.cdiag;
          }
        }
        if (wback) {
          *reinterpret_cast<float4 *>(src) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4 *>(src + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
        if (osplit) {
          float hi[8], lo[8];
          split4(v, hi, lo);
          split4(v + 4, hi + 4, lo + 4);
          if (!t0) {
            st16(S0 + (gi * ld0 + gj) * 2, pack8(hi));
            st16(S1 + (gi * ld1 + gj) * 2, pack8(lo));
          }
        } else {
          if (!t0) st16(S0 + (gi * ld0 + gj) * 2, pack8(v));
          if (S1 && !t1) st16(S1 + (gi * ld1 + gj) * 2, pack8(v));
        }
      }
    };
    if (fast) {
      if (D) {
        // every D chunk of the pass has landed (this also waits for the
        // previous pass's stores); no store of this pass waits on anything
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        row_fast(std::true_type{});
      } else {
        row_fast(std::false_type{});
      }
    } else {
#pragma unroll 1
    for (int q = 0; q < 16; ++q) {
      const int ch = tid + NTHR * q;        // 4096 quads: 64 rows x 64 quads
      const int r = ch >> 6, c4 = (ch & 63) * 4;
      const int64_t gi = m0 + (r >> 5) * 128 + p * 32 + (r & 31);
      const int64_t gj = n0 + c4;
      float *src = stg + srow(r) * SLD + c4;
      float4 v4 = *reinterpret_cast<const float4 *>(src);
      float v[4] = {v4.x, v4.y, v4.z, v4.w};
      if (gi < M) {
        const int nv = (int)min<int64_t>(N - gj, 4);
        float dv[4] = {0.f, 0.f, 0.f, 0.f};
        if (D && nv > 0) load_quad(D, gi * ldd + gj, dv, nv, fd);
        if (dsplit && nv > 0) {
          float dl[4] = {0.f, 0.f, 0.f, 0.f};
          load_quad(D2, gi * ldd + gj, dl, nv, false);
#pragma unroll
          for (int e = 0; e < 4; ++e) dv[e] += dl[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = v[e];
          if (D) x = fmaf(cds, dv[e], x);
          if (diag && gi == gj + e) x += R.cdiag;
          v[e] = x;
        }
        if (wback) *reinterpret_cast<float4 *>(src) = make_float4(v[0], v[1], v[2], v[3]);
        if (nv > 0) {
          if (osplit) {
            float hi[4], lo[4];
            split4(v, hi, lo);
            if (!t0) { store_quad(S0, gi * ld0 + gj, hi, nv, false); store_quad(S1, gi * ld1 + gj, lo, nv, false); }
          } else {
            if (!t0) store_quad(S0, gi * ld0 + gj, v, nv, f0);
            if (S1 && !t1) store_quad(S1, gi * ld1 + gj, v, nv, f1);
          }
        }
      }
    }
    }
    if (col_phase && fast) {
      // transposed / mirror stores of an interior tile: lane l of a wave
      // takes 8-row chunk l % 4 of column c0 + l / 4, so one store
      // instruction writes 64 contiguous bytes to each of 16 output rows
      __syncthreads();
#pragma unroll 2
      for (int q = 0; q < 8; ++q) {
        const int ch = tid + NTHR * q;      // 2048 chunks: 2 row groups x 256 columns x 4
        const int k = ch & 3, c = (ch >> 2) & 255, sg = ch >> 10;
        const float *col = stg + (sg * 32 + k * 8) * SLD + c;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = col[((e + 2 * k) & 7) * SLD];
        const int64_t gi = m0 + sg * 128 + p * 32 + k * 8;
        const int64_t gj = n0 + c;
        if (osplit) {
          float hi[8], lo[8];
          split4(v, hi, lo);
          split4(v + 4, hi + 4, lo + 4);
          if (t0 || mirror) {
            st16(S0 + (gj * ld0 + gi) * 2, pack8(hi));
            st16(S1 + (gj * ld1 + gi) * 2, pack8(lo));
          }
        } else {
          if (t0 || mirror) st16(S0 + (gj * ld0 + gi) * 2, pack8(v));
          if (S1 && (t1 || mirror)) st16(S1 + (gj * ld1 + gi) * 2, pack8(v));
        }
      }
    } else if (col_phase) {
      __syncthreads();
#pragma unroll 1
      for (int q = 0; q < 8; ++q) {
        const int ch = tid + NTHR * q;      // 2048 chunks: 256 columns x 8 row chunks
        const int c = ch & 255, r8 = (ch >> 8) * 8;
        const int64_t gj = n0 + c;
        const int64_t gi = m0 + (r8 >> 5) * 128 + p * 32 + (r8 & 31);
        if (gj >= N) continue;
        const int nv = (int)min<int64_t>(M - gi, 8);
        if (nv <= 0) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = stg[srow(r8 + e) * SLD + c];
        if (osplit) {
          float hi[8], lo[8];
          split4(v, hi, lo);
          split4(v + 4, hi + 4, lo + 4);
          if (t0 || mirror) { store_chunk(S0, gj * ld0 + gi, hi, nv, false); store_chunk(S1, gj * ld1 + gi, lo, nv, false); }
        } else {
          if (t0 || mirror) store_chunk(S0, gj * ld0 + gi, v, nv, f0);
          if (S1 && (t1 || mirror)) store_chunk(S1, gj * ld1 + gi, v, nv, f1);
        }
      }
    }
  }
}

template <bool SPLIT>
__global__ __launch_bounds__(NTHR, 1) void ns_gemm256(GemmArgs args, int ntiles) {
  if (args.skip && *args.skip) return;
#if MUON_XCD_REMAP
  // Workgroup i runs on XCD i % 8.  The tile list is cut into chunks of
  // 8 x 32 tiles; XCD x takes tiles [32 x, 32 x + 32) of each chunk, i.e.
  // about two tile-rows of one problem, so the 32 CUs of an XCD share their
  // operand panels through its L2 while all XCDs stay on the same problem.
  const int xcd = (int)(blockIdx.x % NXCD), slot = (int)(blockIdx.x / NXCD);
  const int t = (slot / XCD_CUS) * (NXCD * XCD_CUS) + xcd * XCD_CUS + slot % XCD_CUS;
  if (t >= ntiles) return;
#else
  const int t = blockIdx.x;
#endif
  gemm_tile<SPLIT>(args.probs, args.ws, args.scales, args.r, args.tiles[t], (int)threadIdx.x);
}

// Dependency waits poll about once a microsecond; past this many polls
// (about four seconds) the item runs anyway and the workgroup stops waiting
// for the rest of the launch, so a fault in the queues shows as wrong
// results (which the parity checks catch) within seconds, never as a hang.
constexpr int kMaxPolls = 1 << 22;

// Persistent grouped launch: one workgroup per CU walks the work queue of
// its XCD, named by the XCC_ID hardware register (bits 3:0), one tile of one
// product of one problem per item.  Every product of a problem runs on the
// XCD its problem was given, so producer and consumer tiles meet in that
// XCD's L2: a finished tile is counted in done[problem] only after every
// wave's stores have reached the L2, and a consumer invalidates its L1
// before it reads.  A queue lists all tiles of a problem's product k before
// any tile of its product k + 1, so an item waits only on items of smaller
// index, which running workgroups hold: every dequeued item completes.
template <bool SPLIT>
__global__ __launch_bounds__(NTHR, 1) void ns_persist(PersistArgs pa) {
  if (pa.skip && *pa.skip) return;
  const int xcd = __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & (PQ_XCDS - 1);
  int32_t *slot = reinterpret_cast<int32_t *>(lds + LDS_SLOT);
  int32_t *head = pa.counters + PQ_PAD * xcd;
  const int q0 = pa.qoff[xcd], qn = pa.qoff[xcd + 1] - q0;
  if (threadIdx.x == 0) slot[0] = atomicAdd(head, 1);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(slot[0]);
  int polls_left = kMaxPolls;  // thread 0's wait budget for the whole launch
  while (cur < qn) {
    const TileDev it = pa.items[q0 + cur];
    const int p = it.prob & PQ_PROB_MASK, k = (int)((uint32_t)it.prob >> PQ_LAUNCH_SHIFT);
    const PLaunch &L = pa.launches[k];
    int32_t *done = pa.counters + PQ_PAD * (PQ_XCDS + p);
    int nxt = 0;
    if (threadIdx.x == 0) {
      nxt = atomicAdd(head, 1);  // the next item, taken now so its latency hides under this tile
      const int need = L.mm_before * pa.ntl[2 * p] + L.mn_before * pa.ntl[2 * p + 1];
      while (polls_left > 0 && __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
        __builtin_amdgcn_s_sleep(2);
        --polls_left;
      }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // the thread index is re-read for every item, so nothing derived from it
    // is hoisted out of the loop and held in registers across the epilogue
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    gemm_tile<SPLIT>(pa.probs, pa.ws, pa.scales, L.r, TileDev{p, it.tm, it.tn}, tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      atomicAdd(done, 1);
      slot[0] = nxt;
    }
    __syncthreads();
    cur = __builtin_amdgcn_readfirstlane(slot[0]);
  }
}

}  // namespace

hipError_t launch_gemm256(const GemmArgs &a, int ntiles, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  const bool split = a.r.nseg > 1 || (a.r.flags & (GF_SPLIT_OUT | GF_D_SPLIT)) != 0;
  auto kern = split ? ns_gemm256<true> : ns_gemm256<false>;
#if MUON_XCD_REMAP
  const int chunk = NXCD * XCD_CUS;
  const int grid = (ntiles + chunk - 1) / chunk * chunk;
#else
  const int grid = ntiles;
#endif
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), 0, s, a, ntiles);
  return hipGetLastError();
}

hipError_t launch_persist(const PersistArgs &a, bool split, hipStream_t s) {
  auto kern = split ? ns_persist<true> : ns_persist<false>;
  hipLaunchKernelGGL(kern, dim3(PQ_XCDS * XCD_CUS), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
