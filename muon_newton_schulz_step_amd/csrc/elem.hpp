// Launchers of the library's kernels (host side).
#pragma once

#include <hip/hip_runtime_api.h>

#include "tables.hpp"

namespace muon {

hipError_t launch_k0(const K0Mat *mats, int nmat, int64_t chunks, bool gbf16, int first, hipStream_t s);
hipError_t launch_k1(const K1Prob *probs, int nprob, int tiles, char *ws, float *partials, float beta, int nesterov,
                     bool gbf16, hipStream_t s);
hipError_t launch_kn(const K1Prob *probs, int nprob, const float *partials, float *scales, float eps, hipStream_t s);
hipError_t launch_k3(const K3Run *runs, int nrun, int64_t chunks, hipStream_t s);
hipError_t launch_kc(const ProbDev *probs, const K1Prob *k1, int nprob, char *ws, const float *scales, hipStream_t s);

// One grouped Newton-Schulz GEMM launch over a tile list.
struct GemmArgs {
  const ProbDev *probs;
  const TileDev *tiles;
  char *ws;
  const float *scales;
  GemmRecipe r;
};
hipError_t launch_gemm(bool bf16_operands, const GemmArgs &a, int ntiles, hipStream_t s);
hipError_t launch_gemm256(const GemmArgs &a, int ntiles, hipStream_t s);

}  // namespace muon
