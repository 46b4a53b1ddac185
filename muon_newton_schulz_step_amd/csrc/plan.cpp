// Host planner (no HIP calls).  See plan.hpp.
#include "elem.hpp"
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>

namespace muon {

namespace {

thread_local std::string g_last_error;

int64_t rup(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int64_t cdiv(int64_t x, int64_t a) { return (x + a - 1) / a; }

constexpr int64_t kAlign = 256;

// Bump allocator over a region.
struct Carver {
  int64_t top = 0;
  int64_t take(int64_t bytes) {
    int64_t o = rup(top, kAlign);
    top = o + bytes;
    return o;
  }
};

double nominal_flops(int method, int steps, double m, double n) {
  if (steps == 0) return 0.0;
  if (method == MUON_NS_STANDARD) return steps * (4.0 * m * m * n + 2.0 * m * m * m);
  // gram: R0 and Q X0 on the m x n side; the m x m chain:
  // steps squarings, steps-1 accumulations of Q, 2(steps-1) for P R P
  double chain = steps + (steps - 1) + 2.0 * (steps - 1);
  return 4.0 * m * m * n + chain * 2.0 * m * m * m;
}

}  // namespace

void set_error(const std::string &msg) { g_last_error = msg; }
const char *last_error() { return g_last_error.c_str(); }

// Owned runs of a matrix: element j of the row-major matrix lands at flat
// index flat_offset + j, partition (f / P), local offset (f % P).
static std::vector<muon_run> make_runs(int32_t mi, int64_t off, int64_t numel, int64_t P) {
  std::vector<muon_run> runs;
  int64_t j = 0;
  while (j < numel) {
    int64_t f = off + j;
    int64_t r = f / P, lo = f % P;
    int64_t n = std::min(numel - j, P - lo);
    runs.push_back(muon_run{mi, (int32_t)r, lo, j, n});
    j += n;
  }
  return runs;
}

// Gram form with a split-bf16 m x m chain (large bf16 blocks): every chain
// matrix is a pair hi = bf16(v), lo = bf16(v - hi), and every chain product
// X Y^T is hi_X hi_Y^T + hi_X lo_Y^T + lo_X hi_Y^T (three K segments of the
// bf16 kernel, fp32 accumulation), about 16 significant bits per entry.
static std::vector<Launch> build_split_gram_schedule(const muon_options &o, bool lean_q) {
  const int T = o.ns_steps;
  std::vector<Launch> S;
  auto base = [&](int rS0, int rS1, int flags, float cd, float cacc, float cdiag) {
    GemmRecipe r;
    std::memset(&r, 0, sizeof(r));
    r.rA = r.rB = r.rD = -1; r.rS0 = (int8_t)rS0; r.rS1 = (int8_t)rS1;
    r.flags = flags; r.cd = cd; r.cacc = cacc; r.cdiag = cdiag;
    r.nseg = 1; r.rA2[0] = r.rA2[1] = r.rB2[0] = r.rB2[1] = -1; r.rD2 = -1;
    return r;
  };
  auto lo_of = [](int hi) {
    switch (hi) {
      case R_MA: return (int)R_MA_LO;
      case R_MB: return (int)R_MB_LO;
      case R_Q0: return (int)R_Q0_LO;
      case R_Q1: return (int)R_Q1_LO;
      default: return (int)R_MT_LO;
    }
  };
  // product X Y^T of two split matrices (hi roles given)
  auto split = [&](GemmRecipe r, int X, int Y) {
    r.rA = (int8_t)X; r.rB = (int8_t)Y;
    r.nseg = 3;
    r.rA2[0] = (int8_t)X; r.rB2[0] = (int8_t)lo_of(Y);
    r.rA2[1] = (int8_t)lo_of(X); r.rB2[1] = (int8_t)Y;
    return r;
  };
  if (T == 0) {
    S.push_back(Launch{Launch::COPY_SCALED, base(-1, -1, 0, 0.f, 0.f, 0.f), false});
    return S;
  }
  const int SP = GF_SYM | GF_SPLIT_OUT;
  // R = s^2 X0 X0^T, stored split
  {
    GemmRecipe r = base(R_MA, R_MA_LO, SP, 0.f, 1.f, 0.f);
    r.rA = r.rB = R_XR0; r.dimK = 1; r.scale_pow = 2;
    S.push_back(Launch{Launch::GEMM_OP, r, false});
  }
  int qcur = -1;
  for (int k = 1; k <= T; ++k) {
    const bool last = (k == T);
    // P = a I + b R + c R R; the first P is Q itself
    const int Pr = (k == 1) ? R_Q0 : R_MB;
    GemmRecipe rp = split(base(Pr, lo_of(Pr), SP | GF_DIAG | GF_D_SPLIT, o.b, o.c, o.a), R_MA, R_MA);
    rp.rD = R_MA; rp.rD2 = R_MA_LO;
    S.push_back(Launch{Launch::GEMM_OP, rp, false});
    if (k == 1) qcur = R_Q0;
    else {
      const int qn = (qcur == R_Q0) ? R_Q1 : R_Q0;
      if (lean_q) {
        // Q <- P Q from the high halves, stored as bf16 only: Q reaches the
        // output through its bf16 value anyway (Y = s Q_hi X0)
        GemmRecipe rq = base(qn, -1, GF_SYM, 0.f, 1.f, 0.f);
        rq.rA = (int8_t)Pr; rq.rB = (int8_t)qcur;
        S.push_back(Launch{Launch::GEMM_OP, rq, false});
      } else {
        S.push_back(Launch{Launch::GEMM_OP, split(base(qn, lo_of(qn), SP, 0.f, 1.f, 0.f), Pr, qcur), false});
      }
      qcur = qn;
    }
    if (!last) {
      S.push_back(Launch{Launch::GEMM_OP, split(base(R_MT, R_MT_LO, SP, 0.f, 1.f, 0.f), Pr, R_MA), false});
      S.push_back(Launch{Launch::GEMM_OP, split(base(R_MA, R_MA_LO, SP, 0.f, 1.f, 0.f), R_MT, Pr), false});
    }
  }
  // Y = s Q X0 with the bf16 high half of Q
  {
    GemmRecipe r = base(R_U, -1, GF_S0_PROBT, 0.f, 1.f, 0.f);
    r.rA = (int8_t)qcur; r.rB = R_XC0; r.dimN = 1; r.scale_pow = 1;
    S.push_back(Launch{Launch::GEMM_OP, r, true});
  }
  return S;
}

// Persistent schedule of a wave's large-tile groups.  The group's problems
// go to the PQ_XCDS queues largest first, each to the queue with the least
// work so far (the wave's problem order is already largest first); a queue
// then lists, launch by launch of the group's schedule, every tile of each
// of its problems in the order of the tile lists.  Every product of a
// problem thus runs on one XCD, after all tiles of its previous product.
static void build_queues(const muon_plan *p, WavePlan &W) {
  const int np = (int)W.probs.size();
  W.pntl.assign(2 * (size_t)np, 0);
  for (int g = PG_BF16_BIG; g < NGROUPS; ++g) {
    const std::vector<Launch> &S = p->schedule[g];
    const std::vector<TileDev> &MM = W.tiles[g][TL_MM256], &MN = W.tiles[g][TL_MN256];
    if (MN.empty() || S.empty() || S.size() > (size_t)PQ_MAX_LAUNCHES) continue;
    bool gemm = true;
    for (const Launch &L : S) gemm = gemm && L.kind == Launch::GEMM_OP;
    if (!gemm) continue;
    std::vector<int64_t> mm0(np, -1), mn0(np, -1);
    for (size_t i = 0; i < MM.size(); ++i) {
      if (mm0[MM[i].prob] < 0) mm0[MM[i].prob] = (int64_t)i;
      ++W.pntl[2 * MM[i].prob];
    }
    for (size_t i = 0; i < MN.size(); ++i) {
      if (mn0[MN[i].prob] < 0) mn0[MN[i].prob] = (int64_t)i;
      ++W.pntl[2 * MN[i].prob + 1];
    }
    double load[PQ_XCDS] = {};
    std::vector<int32_t> xp[PQ_XCDS];
    for (int li = 0; li < np; ++li) {
      if (mn0[li] < 0) continue;
      int best = 0;
      for (int x = 1; x < PQ_XCDS; ++x)
        if (load[x] < load[best]) best = x;
      load[best] += p->probs[W.problems[li]].flops;
      xp[best].push_back(li);
    }
    std::vector<TileDev> &Q = W.pq[g];
    Q.clear();
    for (int x = 0; x < PQ_XCDS; ++x) {
      W.pq_off[g][x] = (int32_t)Q.size();
      for (size_t k = 0; k < S.size(); ++k)
        for (int32_t li : xp[x]) {
          const std::vector<TileDev> &L = S[k].mn ? MN : MM;
          const int64_t a = S[k].mn ? mn0[li] : mm0[li];
          const int32_t n = W.pntl[2 * li + (S[k].mn ? 1 : 0)];
          for (int32_t i = 0; i < n; ++i)
            Q.push_back(TileDev{li | (int32_t)(k << PQ_LAUNCH_SHIFT), L[a + i].tm, L[a + i].tn});
        }
    }
    W.pq_off[g][PQ_XCDS] = (int32_t)Q.size();
    W.pl[g].clear();
    int32_t mmc = 0, mnc = 0;
    for (const Launch &L : S) {
      W.pl[g].push_back(PLaunch{L.r, mmc, mnc});
      (L.mn ? mnc : mmc) += 1;
    }
  }
}

// Launch schedule of one operand class (bf16 = bf16 MFMA operands on the
// m x n side; the Gram form's m x m chain is fp32 in both classes).
static std::vector<Launch> build_schedule(const muon_options &o, bool bf16) {
  const int T = o.ns_steps;
  std::vector<Launch> S;
  auto recipe = [](int rA, int rB, int rD, int rS0, int rS1, int dM, int dN, int dK, int flags,
                   float cd, float cacc, float cdiag, int sp) {
    GemmRecipe r;
    std::memset(&r, 0, sizeof(r));
    r.rA = (int8_t)rA; r.rB = (int8_t)rB; r.rD = (int8_t)rD; r.rS0 = (int8_t)rS0; r.rS1 = (int8_t)rS1;
    r.dimM = (int8_t)dM; r.dimN = (int8_t)dN; r.dimK = (int8_t)dK;
    r.flags = flags; r.cd = cd; r.cacc = cacc; r.cdiag = cdiag; r.scale_pow = sp;
    r.nseg = 1; r.rA2[0] = r.rA2[1] = r.rB2[0] = r.rB2[1] = -1; r.rD2 = -1;
    return r;
  };
  if (T == 0) {
    S.push_back(Launch{Launch::COPY_SCALED, recipe(-1, -1, -1, -1, -1, 0, 0, 0, 0, 0.f, 0.f, 0.f, 0), false});
    return S;
  }
  const int opf32 = bf16 ? 0 : (GF_S0_F32 | GF_S1_F32);
  const int dopf32 = bf16 ? 0 : GF_D_F32;
  const Launch::Kind OPK = bf16 ? Launch::GEMM_OP : Launch::GEMM_F32;
  if (o.method == MUON_NS_STANDARD) {
    // Each step X <- a X + (b A + c A^2) X is evaluated as C X with
    // C = a I + b A + c A^2 (equal in exact arithmetic).  Rounding C rather
    // than b A + c A^2 to the operand dtype avoids the cancellation between
    // a X and (b A + c A^2) X once the singular values approach 1.
    for (int t = 0; t < T; ++t) {
      int cur = t & 1, nxt = cur ^ 1;
      int XR = cur ? R_XR1 : R_XR0, XC = cur ? R_XC1 : R_XC0;
      int XRn = nxt ? R_XR1 : R_XR0, XCn = nxt ? R_XC1 : R_XC0;
      // A = s^2 X X^T
      S.push_back(Launch{OPK, recipe(XR, XR, -1, R_MA, -1, 0, 0, 1, GF_SYM | opf32, 0.f, 1.f, 0.f,
                                     t == 0 ? 2 : 0), false});
      // C = a I + b A + c A A
      S.push_back(Launch{OPK, recipe(R_MA, R_MA, R_MA, R_MB, -1, 0, 0, 0, GF_SYM | GF_DIAG | opf32 | dopf32,
                                     o.b, o.c, o.a, 0), false});
      // X' = s C X
      if (t < T - 1)
        S.push_back(Launch{OPK, recipe(R_MB, XC, -1, XRn, XCn, 0, 1, 0, GF_S1_TRANS | opf32, 0.f, 1.f, 0.f,
                                       t == 0 ? 1 : 0), true});
      else
        S.push_back(Launch{OPK, recipe(R_MB, XC, -1, R_U, -1, 0, 1, 0, GF_S0_PROBT | (bf16 ? 0 : GF_S0_F32), 0.f,
                                       1.f, 0.f, t == 0 ? 1 : 0), true});
    }
    return S;
  }
  // Gram form.  The m x m chain is fp32.
  const int F = GF_S0_F32 | GF_S1_F32 | GF_D_F32;
  S.push_back(Launch{OPK, recipe(R_XR0, R_XR0, -1, R_MA, -1, 0, 0, 1, GF_SYM | GF_S0_F32, 0.f, 1.f, 0.f, 2),
                     false});
  int qcur = -1;
  for (int k = 1; k <= T; ++k) {
    const bool last = (k == T);
    // P = a I + b R + c R R
    int s1 = -1, fl = GF_SYM | GF_DIAG | F;
    if (k == 1) {
      if (last && bf16) { s1 = R_QB; fl &= ~GF_S1_F32; }
      else s1 = R_Q0;
      qcur = R_Q0;
    }
    S.push_back(Launch{Launch::GEMM_F32, recipe(R_MA, R_MA, R_MA, R_MB, s1, 0, 0, 0, fl, o.b, o.c, o.a, 0),
                       false});
    if (k >= 2) {
      int qn = (qcur == R_Q0) ? R_Q1 : R_Q0;
      int s1b = -1, flb = GF_SYM | F;
      if (last && bf16) { s1b = R_QB; flb &= ~GF_S1_F32; }
      S.push_back(Launch{Launch::GEMM_F32, recipe(R_MB, qcur, -1, qn, s1b, 0, 0, 0, flb, 0.f, 1.f, 0.f, 0),
                         false});
      qcur = qn;
    }
    if (!last) {
      S.push_back(Launch{Launch::GEMM_F32, recipe(R_MB, R_MA, -1, R_MT, -1, 0, 0, 0, GF_SYM | F, 0.f, 1.f, 0.f, 0),
                         false});
      S.push_back(Launch{Launch::GEMM_F32, recipe(R_MT, R_MB, -1, R_MA, -1, 0, 0, 0, GF_SYM | F, 0.f, 1.f, 0.f, 0),
                         false});
    }
  }
  // Y = s Q X0
  int qa = bf16 ? R_QB : qcur;
  S.push_back(Launch{OPK, recipe(qa, R_XC0, -1, R_U, -1, 0, 1, 0, GF_S0_PROBT | (bf16 ? 0 : GF_S0_F32), 0.f, 1.f,
                                 0.f, 1), true});
  return S;
}

muon_status build_plan(muon_plan *p) {
  const muon_options &o = p->opt;
  const int64_t P = p->layout.partition_numel;
  const int32_t nmat = (int32_t)p->mats.size();
  const bool bf16 = o.precision == MUON_PREC_BF16;
  const bool standard = o.method == MUON_NS_STANDARD;
  const int upar = (standard && o.ns_steps > 0) ? (o.ns_steps & 1) : 1;

  // problems, runs, shape scales, operand class
  p->probs.clear();
  for (int32_t i = 0; i < nmat; ++i) {
    auto &M = p->mats[i];
    const int64_t rows = M.desc.rows, cols = M.desc.cols;
    M.heads = M.desc.num_heads > 1 ? M.desc.num_heads : 1;
    M.hr = rows / M.heads;
    M.scale = (float)std::sqrt(std::max(1.0, (double)rows / (double)cols));
    M.runs = make_runs(i, M.desc.flat_offset, rows * cols, P);
    M.prob0 = (int32_t)p->probs.size();
    M.ops32 = !bf16 || std::min<int64_t>(M.hr, cols) < BF16_MIN_M;
    M.elem = M.ops32 ? 4 : 2;
    M.ldc = rup(cols, 8);
    M.ldhr = rup(M.hr, 8);
    for (int32_t h = 0; h < M.heads; ++h) {
      ProblemPlan q;
      q.matrix = i; q.head = h;
      q.tall = M.hr > cols;
      q.m = (int32_t)std::min<int64_t>(M.hr, cols);
      q.n = (int32_t)std::max<int64_t>(M.hr, cols);
      q.ldm = rup(q.m, 8);
      q.flops = nominal_flops(o.method, o.ns_steps, q.m, q.n);
      std::fill(q.mm_off, q.mm_off + 6, -1);
      std::fill(q.lo_off, q.lo_off + 5, -1);
      p->probs.push_back(q);
    }
  }

  // Index ranges of the device tables: tile coordinates are int16, tile,
  // K1-tile and chunk indices int32 (also the grid sizes of the launches).
  // A group beyond them is refused here rather than wrapped on the device.
  {
    int64_t k1_total = 0, k3_total = 0, tiles_total = 0;
    for (const ProblemPlan &q : p->probs) {
      const int64_t tm = cdiv(q.m, GEMM_TILE), tn = cdiv(q.n, GEMM_TILE);
      if (tn > INT16_MAX) {
        set_error("matrix " + std::to_string(q.matrix) + ": a side of " + std::to_string(q.n) +
                  " elements needs more than 32767 GEMM tiles");
        return MUON_ERR_UNSUPPORTED;
      }
      const auto &M = p->mats[q.matrix];
      k1_total += cdiv(M.hr, K1_TILE) * cdiv(M.desc.cols, K1_TILE);
      tiles_total += tm * tn + tm * (tm + 1) / 2;
    }
    for (const auto &M : p->mats)
      for (const muon_run &r : M.runs) k3_total += cdiv(r.length, std::min(K3_CHUNK, KA_CHUNK));
    int64_t k0_total = 0;
    for (const auto &M : p->mats) k0_total += cdiv(M.desc.rows * M.desc.cols, K0_CHUNK);
    if (k1_total > INT32_MAX || k3_total > INT32_MAX || k0_total > INT32_MAX || tiles_total > INT32_MAX ||
        (int64_t)p->probs.size() > INT32_MAX) {
      set_error("group too large for the launch tables (more than 2^31-1 tiles or chunks)");
      return MUON_ERR_UNSUPPORTED;
    }
  }

  // per-matrix and per-problem data bytes
  auto matrix_bytes = [&](const MatrixPlan &M) {
    int64_t orig = rup(M.desc.rows * M.ldc * M.elem, kAlign);
    int64_t trans = rup(M.heads * M.desc.cols * M.ldhr * M.elem, kAlign);
    return 2 * orig + (standard ? 2 : 1) * trans;
  };
  auto split_chain = [&](const ProblemPlan &q) {
    return !standard && !p->mats[q.matrix].ops32 && q.m >= BIG_TILE_MIN_M;
  };
  // blocks whose whole iteration runs in one workgroup: no m x m buffers
  auto fused = [&](const ProblemPlan &q) {
    return o.ns_steps > 0 && !p->mats[q.matrix].ops32 && q.m <= HEAD_MAX_M;
  };
  // Parity of the original-layout X copy that U aliases: one the matrix's
  // last Newton-Schulz reads do not touch.  The fused blocks read only
  // parity 0 (the workgroups of a matrix's head blocks run at different
  // times, so U may not alias anything any of them reads).
  auto u_parity = [&](const MatrixPlan &M) { return fused(p->probs[M.prob0]) ? 1 : upar; };
  auto problem_bytes = [&](const ProblemPlan &q) {
    const int64_t e = p->mats[q.matrix].elem;
    int64_t mm = q.m * q.ldm;
    if (fused(q)) return (int64_t)0;
    if (standard) return 2 * rup(mm * e, kAlign);
    if (split_chain(q)) return 10 * rup(mm * 2, kAlign);
    return 5 * rup(mm * 4, kAlign) + (e == 2 ? rup(mm * 2, kAlign) : 0);
  };

  // waves: matrices in order, cut when the cap would be exceeded
  p->waves.clear();
  {
    WavePlan cur;
    for (int32_t i = 0; i < nmat; ++i) {
      auto &M = p->mats[i];
      int64_t b = matrix_bytes(M);
      for (int32_t h = 0; h < M.heads; ++h) b += problem_bytes(p->probs[M.prob0 + h]);
      b += kAlign * (4 + 6 * M.heads);
      if (!cur.matrices.empty() && o.max_inflight_bytes && cur.data_bytes + b > (int64_t)o.max_inflight_bytes) {
        p->waves.push_back(std::move(cur));
        cur = WavePlan();
      }
      cur.matrices.push_back(i);
      cur.data_bytes += b;
    }
    p->waves.push_back(std::move(cur));
  }

  p->schedule[PG_F32] = build_schedule(o, false);
  p->schedule[PG_BF16] = build_schedule(o, true);
  p->schedule[PG_BF16_BIG] = standard ? p->schedule[PG_BF16] : build_split_gram_schedule(o, false);
  p->schedule[PG_BF16_LEAN] = standard ? p->schedule[PG_BF16] : build_split_gram_schedule(o, true);

  int64_t max_k1 = 0, max_probs = 0, max_data = 0, nparts = 0;
  for (size_t w = 0; w < p->waves.size(); ++w) {
    WavePlan &W = p->waves[w];
    Carver dat;
    for (int32_t i : W.matrices) {
      MatrixPlan &M = p->mats[i];
      const int64_t e = M.elem;
      M.wave = (int32_t)w;
      int64_t orig = M.desc.rows * M.ldc * e;
      int64_t trans = M.heads * M.desc.cols * M.ldhr * e;
      M.orig_off[0] = dat.take(orig);
      M.orig_off[1] = dat.take(orig);
      M.trans_off[0] = dat.take(trans);
      M.trans_off[1] = standard ? dat.take(trans) : -1;
      for (int32_t h = 0; h < M.heads; ++h) {
        ProblemPlan &q = p->probs[M.prob0 + h];
        int64_t mm = q.m * q.ldm;
        std::fill(q.lo_off, q.lo_off + 5, -1);
        std::fill(q.mm_off, q.mm_off + 6, -1);
        if (fused(q)) {
          // R, P and Q stay on the CU
        } else if (standard) {
          q.mm_off[0] = dat.take(mm * e);
          q.mm_off[1] = dat.take(mm * e);
        } else if (split_chain(q)) {
          for (int r = 0; r < 5; ++r) q.mm_off[r] = dat.take(mm * 2);
          for (int r = 0; r < 5; ++r) q.lo_off[r] = dat.take(mm * 2);
          q.mm_off[5] = -1;
        } else {
          for (int r = 0; r < 5; ++r) q.mm_off[r] = dat.take(mm * 4);
          q.mm_off[5] = e == 2 ? dat.take(mm * 2) : -1;
        }
        W.problems.push_back(M.prob0 + h);
      }
    }
    W.data_bytes = dat.top;
    max_data = std::max(max_data, dat.top);
    // LPT: largest problems first (stable, so equal problems keep group order)
    std::stable_sort(W.problems.begin(), W.problems.end(),
                     [&](int32_t a, int32_t b) { return p->probs[a].flops > p->probs[b].flops; });
    max_probs = std::max<int64_t>(max_probs, (int64_t)W.problems.size());
  }

  Carver tab;
  for (size_t w = 0; w < p->waves.size(); ++w) {
    WavePlan &W = p->waves[w];
    W.probs.clear(); W.k1.clear(); W.runs.clear(); W.run_src.clear(); W.k1_matrix.clear();
    for (int g = 0; g < NGROUPS; ++g)
      for (int l = 0; l < NLISTS; ++l) W.tiles[g][l].clear();
    int32_t k1t = 0;
    for (size_t li = 0; li < W.problems.size(); ++li) {
      const ProblemPlan &q = p->probs[W.problems[li]];
      const MatrixPlan &M = p->mats[q.matrix];
      const int64_t e = M.elem;
      ProbDev d;
      std::memset(&d, 0, sizeof(d));
      for (int r = 0; r < NROLES; ++r) { d.off[r] = -1; d.ld[r] = 0; }
      d.m = q.m; d.n = q.n; d.matrix = q.matrix; d.flags = q.tall ? PF_TALL : 0;
      // two copies of X: original layout (rows of the block) and transposed
      for (int par = 0; par < 2; ++par) {
        int64_t oo = M.orig_off[par] + (int64_t)q.head * M.hr * M.ldc * e;
        int64_t to = M.trans_off[par] < 0 ? -1 : M.trans_off[par] + (int64_t)q.head * M.desc.cols * M.ldhr * e;
        int rXR = par ? R_XR1 : R_XR0, rXC = par ? R_XC1 : R_XC0;
        if (!q.tall) {
          d.off[rXR] = oo; d.ld[rXR] = (int32_t)M.ldc;
          d.off[rXC] = to; d.ld[rXC] = (int32_t)M.ldhr;
        } else {
          d.off[rXR] = to; d.ld[rXR] = (int32_t)M.ldhr;
          d.off[rXC] = oo; d.ld[rXC] = (int32_t)M.ldc;
        }
      }
      for (int r = 0; r < 6; ++r) {
        d.off[R_MA + r] = q.mm_off[r];
        d.ld[R_MA + r] = (int32_t)q.ldm;
      }
      for (int r = 0; r < 5; ++r) {
        d.off[R_MA_LO + r] = q.lo_off[r];
        d.ld[R_MA_LO + r] = (int32_t)q.ldm;
      }
      // U: dense original orientation.  It aliases the original-layout copy
      // of X that the last Newton-Schulz launch does not read: parity T&1 of
      // the standard form (the final launch reads parity (T-1)&1), parity 1
      // for the Gram form and for zero steps (both read only parity 0).
      d.off[R_U] = M.orig_off[u_parity(M)] + (int64_t)q.head * M.hr * M.desc.cols * e;
      d.ld[R_U] = (int32_t)M.desc.cols;
      W.probs.push_back(d);

      K1Prob k;
      std::memset(&k, 0, sizeof(k));
      k.row0 = (int64_t)q.head * M.hr;
      k.cols = M.desc.cols;
      k.hr = (int32_t)M.hr;
      k.orig_off = M.orig_off[0] + (int64_t)q.head * M.hr * M.ldc * e;
      k.orig_ld = (int32_t)M.ldc;
      k.trans_off = M.trans_off[0] + (int64_t)q.head * M.desc.cols * M.ldhr * e;
      k.trans_ld = (int32_t)M.ldhr;
      k.tiles_c = (int32_t)cdiv(M.desc.cols, K1_TILE);
      k.ntiles = (int32_t)(cdiv(M.hr, K1_TILE) * k.tiles_c);
      k.tile0 = k1t;
      k.xbf16 = M.ops32 ? 0 : 1;
      k1t += k.ntiles;
      W.k1.push_back(k);
      W.k1_matrix.push_back(q.matrix);

      const int grp = M.ops32 ? PG_F32
                      : fused(q) ? PG_HEAD
                      : q.m < BIG_TILE_MIN_M ? PG_BF16
                      : (!standard && q.m >= GRAM_LEAN_MIN_M) ? PG_BF16_LEAN : PG_BF16_BIG;
      // Tiles of a problem in 4 x 8 blocks (block-row-major, row-major inside
      // a block): the large-tile kernel hands each XCD 32 consecutive
      // entries, i.e. one block, whose 12 operand panels its L2 then shares.
      auto add_tiles = [&](int tile, int lmm, int lmn) {
        const int64_t tmn = cdiv(q.m, tile), tnn = cdiv(q.n, tile);
        constexpr int64_t BR = 4, BC = 8;
        for (int64_t A0 = 0; A0 < tmn; A0 += BR)
          for (int64_t B0 = 0; B0 < tmn; B0 += BC)
            for (int64_t a = A0; a < std::min(A0 + BR, tmn); ++a)
              for (int64_t b = std::max(B0, a); b < std::min(B0 + BC, tmn); ++b)
                W.tiles[grp][lmm].push_back(TileDev{(int32_t)li, (int16_t)a, (int16_t)b});
        for (int64_t A0 = 0; A0 < tmn; A0 += BR)
          for (int64_t B0 = 0; B0 < tnn; B0 += BC)
            for (int64_t a = A0; a < std::min(A0 + BR, tmn); ++a)
              for (int64_t b = B0; b < std::min(B0 + BC, tnn); ++b)
                W.tiles[grp][lmn].push_back(TileDev{(int32_t)li, (int16_t)a, (int16_t)b});
      };
      if (grp == PG_HEAD) W.tiles[grp][TL_MN128].push_back(TileDev{(int32_t)li, 0, 0});
      else add_tiles(GEMM_TILE, TL_MM128, TL_MN128);
      if (grp >= PG_BF16_BIG) add_tiles(BIG_TILE, TL_MM256, TL_MN256);
    }
    W.k1_tiles = k1t;
    max_k1 = std::max<int64_t>(max_k1, k1t);
    if (o.schedule == MUON_SCHED_PERSISTENT) build_queues(p, W);
    int64_t ch = 0;
    for (int32_t i : W.matrices) {
      const MatrixPlan &M = p->mats[i];
      for (const muon_run &r : M.runs) {
        K3Run k;
        std::memset(&k, 0, sizeof(k));
        k.first = r.first; k.length = r.length; k.chunk0 = ch; k.scale = M.scale;
        k.src_bf16 = M.ops32 ? 0 : 1;
        ch += cdiv(r.length, K3_CHUNK);
        W.runs.push_back(k);
        W.run_src.push_back(r);
      }
    }
    W.k3_chunks = ch;
    W.k3_base = nparts;
    nparts += ch;
    W.off_prob = tab.take((int64_t)W.probs.size() * sizeof(ProbDev));
    W.off_k1 = tab.take((int64_t)W.k1.size() * sizeof(K1Prob));
    for (int g = 0; g < NGROUPS; ++g)
      for (int l = 0; l < NLISTS; ++l) W.off_tiles[g][l] = tab.take((int64_t)W.tiles[g][l].size() * sizeof(TileDev));
    W.off_runs = tab.take((int64_t)W.runs.size() * sizeof(K3Run));
    W.off_pntl = tab.take((int64_t)W.pntl.size() * 4);
    for (int g = 0; g < NGROUPS; ++g) {
      if (W.pq[g].empty()) continue;
      W.off_pq[g] = tab.take((int64_t)W.pq[g].size() * sizeof(TileDev));
      W.off_pl[g] = tab.take((int64_t)W.pl[g].size() * sizeof(PLaunch));
      // the counters stay zero in the serialized tables, so every upload
      // clears them
      W.off_pcnt[g] = tab.take((int64_t)(PQ_XCDS + W.probs.size()) * PQ_PAD * 4);
    }
  }
  // the accumulation and scatter tables reuse the head of the table region
  int64_t scatter_runs = 0;
  for (auto &M : p->mats) scatter_runs += (int64_t)M.runs.size();
  p->k0_table_bytes = std::max<int64_t>(rup(nmat * (int64_t)sizeof(K0Mat), kAlign),
                                         std::max(rup(scatter_runs * (int64_t)sizeof(K3Run), kAlign),
                                                  rup(scatter_runs * (int64_t)sizeof(KARun), kAlign)));
  p->tables_bytes = std::max(rup(tab.top, kAlign), p->k0_table_bytes);
  p->max_k1_tiles = max_k1;
  p->max_probs = max_probs;
  Carver ws;
  ws.take(p->tables_bytes);
  p->partials_off = ws.take(std::max<int64_t>(max_k1, 1) * 4);
  p->scales_off = ws.take(std::max<int64_t>(max_probs, 1) * 4);
  p->nparts_n = nparts;
  p->nparts_off = ws.take(std::max<int64_t>(nparts, 1) * 4);
  p->nc_off = ws.take(2 * 4);
  p->nl1_off = ws.take(std::max<int64_t>((nparts + kNormSpan - 1) / kNormSpan, 1) * 8);
  p->data_off = ws.take(max_data);
  p->ws_bytes = rup(ws.top, kAlign);
  // absolute offsets inside the workspace
  for (auto &M : p->mats) M.u_off = p->data_off + M.orig_off[u_parity(M)];
  for (auto &W : p->waves) {
    for (auto &d : W.probs)
      for (int r = 0; r < NROLES; ++r)
        if (d.off[r] >= 0) d.off[r] += p->data_off;
    for (auto &k : W.k1) { k.orig_off += p->data_off; k.trans_off += p->data_off; }
  }
  // serialize (an empty table has no data pointer to copy from)
  p->host_tables.assign(p->tables_bytes, 0);
  auto put = [&](int64_t off, const auto &v) {
    if (!v.empty()) std::memcpy(p->host_tables.data() + off, v.data(), v.size() * sizeof(v[0]));
  };
  for (auto &W : p->waves) {
    put(W.off_prob, W.probs);
    put(W.off_k1, W.k1);
    for (int g = 0; g < NGROUPS; ++g)
      for (int l = 0; l < NLISTS; ++l) put(W.off_tiles[g][l], W.tiles[g][l]);
    put(W.off_runs, W.runs);
    put(W.off_pntl, W.pntl);
    for (int g = 0; g < NGROUPS; ++g) {
      put(W.off_pq[g], W.pq[g]);
      put(W.off_pl[g], W.pl[g]);
    }
  }
  return MUON_OK;
}

}  // namespace muon

using muon::set_error;

extern "C" {

muon_status muon_default_options(muon_options *out) {
  if (!out) { set_error("muon_default_options: out is NULL"); return MUON_ERR_INVALID_ARG; }
  std::memset(out, 0, sizeof(*out));
  out->beta = 0.95f;
  out->nesterov = 1;
  out->method = MUON_NS_STANDARD;
  out->ns_steps = 5;
  out->a = 3.4445f; out->b = -4.7750f; out->c = 2.0315f;
  out->eps = 1e-7f;
  out->precision = MUON_PREC_BF16;
  out->grad_dtype = MUON_DT_BF16;
  out->max_inflight_bytes = MUON_DEFAULT_INFLIGHT_BYTES;
  out->schedule = MUON_SCHED_LAUNCHES;
  return MUON_OK;
}

muon_status muon_plan_create(muon_plan **out, const muon_matrix *mats, int32_t n, const muon_options *opt,
                             const muon_layout *layout) {
  if (!out || !mats || !opt || !layout) { set_error("muon_plan_create: NULL argument"); return MUON_ERR_INVALID_ARG; }
  *out = nullptr;
  if (n < 1) { set_error("muon_plan_create: empty group"); return MUON_ERR_INVALID_ARG; }
  if (opt->method != MUON_NS_STANDARD && opt->method != MUON_NS_GRAM) {
    set_error("unknown Newton-Schulz method"); return MUON_ERR_INVALID_ARG;
  }
  if (opt->precision != MUON_PREC_FP32 && opt->precision != MUON_PREC_BF16) {
    set_error("unknown Newton-Schulz precision"); return MUON_ERR_INVALID_ARG;
  }
  if (opt->grad_dtype != MUON_DT_FP32 && opt->grad_dtype != MUON_DT_BF16) {
    set_error("unknown gradient dtype"); return MUON_ERR_INVALID_ARG;
  }
  if (opt->ns_steps < 0 || opt->ns_steps > 64) { set_error("ns_steps must be in [0, 64]"); return MUON_ERR_INVALID_ARG; }
  if (!(opt->beta >= 0.0f && opt->beta < 1.0f)) { set_error("beta must be in [0, 1)"); return MUON_ERR_INVALID_ARG; }
  if (opt->nesterov != 0 && opt->nesterov != 1) { set_error("nesterov must be 0 or 1"); return MUON_ERR_INVALID_ARG; }
  if (opt->schedule != MUON_SCHED_LAUNCHES && opt->schedule != MUON_SCHED_PERSISTENT) {
    set_error("unknown Newton-Schulz schedule"); return MUON_ERR_INVALID_ARG;
  }
  if (opt->reserved != 0) { set_error("options: reserved must be 0"); return MUON_ERR_INVALID_ARG; }
  if (!std::isfinite(opt->a) || !std::isfinite(opt->b) || !std::isfinite(opt->c) || !(opt->eps >= 0.0f) ||
      !std::isfinite(opt->eps)) {
    set_error("coefficients must be finite and eps >= 0"); return MUON_ERR_INVALID_ARG;
  }
  if (layout->partition_numel < 1 || layout->num_partitions < 1 || layout->reserved != 0) {
    set_error("layout needs partition_numel >= 1, num_partitions >= 1, reserved == 0");
    return MUON_ERR_INVALID_ARG;
  }
  const int64_t P = layout->partition_numel, R = layout->num_partitions;
  if (P > INT64_MAX / R) { set_error("layout too large"); return MUON_ERR_LAYOUT; }
  const int64_t total = P * R;
  std::vector<std::pair<int64_t, int64_t>> ranges;
  for (int32_t i = 0; i < n; ++i) {
    const muon_matrix &M = mats[i];
    if (M.rows < 1 || M.cols < 1 || M.rows > INT32_MAX / 2 || M.cols > INT32_MAX / 2) {
      set_error("matrix " + std::to_string(i) + ": rows and cols must be in [1, 2^30)");
      return MUON_ERR_INVALID_ARG;
    }
    if (M.reserved != 0) { set_error("matrix " + std::to_string(i) + ": reserved must be 0"); return MUON_ERR_INVALID_ARG; }
    if (M.num_heads < 0) { set_error("matrix " + std::to_string(i) + ": num_heads < 0"); return MUON_ERR_INVALID_ARG; }
    if (M.num_heads > 1 && M.rows % M.num_heads != 0) {
      set_error("matrix " + std::to_string(i) + ": num_heads does not divide rows");
      return MUON_ERR_UNSUPPORTED;
    }
    const int64_t numel = M.rows * M.cols;
    if (M.flat_offset < 0 || M.flat_offset > total || numel > total - M.flat_offset) {
      set_error("matrix " + std::to_string(i) + ": flat range leaves the partitions");
      return MUON_ERR_LAYOUT;
    }
    ranges.push_back({M.flat_offset, M.flat_offset + numel});
  }
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second) { set_error("flat ranges of two matrices overlap"); return MUON_ERR_LAYOUT; }

  muon_plan *p = new (std::nothrow) muon_plan();
  if (!p) { set_error("out of host memory"); return MUON_ERR_INVALID_ARG; }
  p->opt = *opt;
  p->layout = *layout;
  p->mats.resize(n);
  for (int32_t i = 0; i < n; ++i) p->mats[i].desc = mats[i];
  muon_status st = muon::build_plan(p);
  if (st != MUON_OK) { delete p; return st; }
  p->stats.waves = p->waves.size();
  p->patch_host.resize(p->host_tables.size());
  p->ranges.reserve(2 * (size_t)n + (size_t)layout->num_partitions + 4);
  *out = p;
  return MUON_OK;
}

muon_status muon_plan_workspace_bytes(const muon_plan *p, size_t *bytes) {
  if (!p || !bytes) { set_error("muon_plan_workspace_bytes: NULL argument"); return MUON_ERR_INVALID_ARG; }
  *bytes = (size_t)p->ws_bytes;
  return MUON_OK;
}

muon_status muon_plan_stats(const muon_plan *p, muon_stats *out) {
  if (!p || !out) { set_error("muon_plan_stats: NULL argument"); return MUON_ERR_INVALID_ARG; }
  *out = p->stats;
  return MUON_OK;
}

muon_status muon_plan_runs(const muon_plan *p, int32_t matrix, muon_run *out, int32_t cap, int32_t *count) {
  if (!p || !count || cap < 0 || (cap > 0 && !out)) { set_error("muon_plan_runs: bad argument"); return MUON_ERR_INVALID_ARG; }
  if (matrix < 0 || matrix >= (int32_t)p->mats.size()) { set_error("muon_plan_runs: matrix out of range"); return MUON_ERR_INVALID_ARG; }
  const auto &runs = p->mats[matrix].runs;
  *count = (int32_t)runs.size();
  for (int32_t i = 0; i < cap && i < (int32_t)runs.size(); ++i) out[i] = runs[i];
  return MUON_OK;
}

muon_status muon_plan_problems(const muon_plan *p, muon_problem_info *out, int32_t cap, int32_t *count) {
  if (!p || !count || cap < 0 || (cap > 0 && !out)) { set_error("muon_plan_problems: bad argument"); return MUON_ERR_INVALID_ARG; }
  *count = (int32_t)p->probs.size();
  for (int32_t i = 0; i < cap && i < (int32_t)p->probs.size(); ++i) {
    const auto &q = p->probs[i];
    out[i] = muon_problem_info{q.matrix, q.head, q.m, q.n, q.tall ? 1 : 0, p->mats[q.matrix].wave, q.flops};
  }
  return MUON_OK;
}

const char *muon_status_string(muon_status s) {
  switch (s) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_LAYOUT: return "MUON_ERR_LAYOUT";
    case MUON_ERR_ALIAS: return "MUON_ERR_ALIAS";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
  }
  return "unknown muon_status";
}

const char *muon_last_error(void) { return muon::last_error(); }

}  // extern "C"
