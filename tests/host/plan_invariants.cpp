// Host-only check of the planner's invariants, built with AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_planner_sanitized.py compiles it
// with g++ together with csrc/plan.cpp; no HIP call is made).
//
// Random groups (shapes from 1 x 1 to a few thousand, head splits, both
// forms, both precisions, 0..5 steps, 1..5 partitions, packed or aligned
// layouts, workspace caps that cut waves) are planned, and every table the
// kernels will read is checked against the bounds they rely on:
//   - every role buffer of every problem lies inside the workspace data
//     region, and no two buffers of a wave overlap (the dense output U is
//     checked to lie inside the X copy it aliases instead);
//   - every tile of every tile list lies inside its problem, symmetric lists
//     hold upper-triangle tiles only, and 256-tile lists belong to problems
//     with m >= 256; the blocks fused into one workgroup each are exactly
//     the bf16 blocks with 64 <= m <= 128 (at least one step), listed once,
//     with no m x m buffer, no tile elsewhere and U apart from what they read;
//   - the persistent queues hold exactly the tiles of every launch of the
//     large-tile schedules, each problem in one queue with its launches in
//     order, with the counts the kernel's dependency test reads and zero
//     counters, spread over the queues as LPT spreads them;
//   - every K1 entry covers its block, every owned run lies inside its
//     matrix and its partition, the chunk prefixes count the chunks exactly;
//   - the serialized tables fit their region and the scratch sums follow it.
// Invalid groups are refused with the documented status.  Exit status 0 and
// the line "plan invariants ok" mean every check held.
#include <algorithm>
#include <array>
#include <cstring>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "muon.h"
#include "plan.hpp"

using namespace muon;

namespace {

int g_fail = 0;
uint64_t g_queued = 0;  // plans with at least one persistent queue

void fail(const std::string &what, uint64_t it) {
  if (g_fail < 20) std::fprintf(stderr, "iteration %llu: %s\n", (unsigned long long)it, what.c_str());
  ++g_fail;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Span {
  int64_t lo, hi;
  int prob, role;
};

// Element size and shape (rows, cols, ld) of role r of problem d, as the
// kernels address it; false if the role is unused.
bool role_shape(const muon_plan *p, const ProbDev &d, int r, int64_t *bytes) {
  if (d.off[r] < 0) return false;
  const MatrixPlan &M = p->mats[d.matrix];
  const bool standard = p->opt.method == MUON_NS_STANDARD;
  const int64_t op = M.elem;
  const int64_t m = d.m, n = d.n, ld = d.ld[r];
  int64_t rows = 0, cols = 0, e = op;
  switch (r) {
    case R_XR0: case R_XR1: rows = m; cols = n; break;
    case R_XC0: case R_XC1: rows = n; cols = m; break;
    case R_U:
      rows = (d.flags & PF_TALL) ? n : m;
      cols = (d.flags & PF_TALL) ? m : n;
      break;
    case R_QB: rows = m; cols = m; e = 2; break;
    default: {
      rows = m; cols = m;
      const bool split = !standard && !M.ops32 && m >= BIG_TILE_MIN_M;
      if (standard) e = op;
      else e = split ? 2 : 4;
    }
  }
  if (ld < cols) return false;
  *bytes = ((rows - 1) * ld + cols) * e;
  return true;
}

void check_plan(const muon_plan *p, uint64_t it) {
  const int64_t ws = p->ws_bytes;
  if (p->tables_bytes > p->partials_off || p->partials_off > p->scales_off || p->data_off > ws)
    fail("workspace regions out of order", it);
  if ((int64_t)p->host_tables.size() != p->tables_bytes) fail("serialized tables size", it);
  if (p->patch_host.size() != p->host_tables.size()) fail("patch buffer size", it);
  const int64_t P = p->layout.partition_numel;
  int64_t nparts = 0;
  for (const WavePlan &W : p->waves) {
    // tables inside their region
    auto in_tables = [&](int64_t off, int64_t bytes) { return off >= 0 && off + bytes <= p->tables_bytes; };
    if (!in_tables(W.off_prob, (int64_t)(W.probs.size() * sizeof(ProbDev))) ||
        !in_tables(W.off_k1, (int64_t)(W.k1.size() * sizeof(K1Prob))) ||
        !in_tables(W.off_runs, (int64_t)(W.runs.size() * sizeof(K3Run))))
      fail("a table leaves the table region", it);
    for (int g = 0; g < NGROUPS; ++g)
      for (int l = 0; l < NLISTS; ++l)
        if (!in_tables(W.off_tiles[g][l], (int64_t)(W.tiles[g][l].size() * sizeof(TileDev))))
          fail("a tile list leaves the table region", it);
    // role buffers
    std::vector<Span> spans;
    for (size_t pi = 0; pi < W.probs.size(); ++pi) {
      const ProbDev &d = W.probs[pi];
      if (d.m < 1 || d.n < d.m) fail("problem not in the wide orientation", it);
      for (int r = 0; r < NROLES; ++r) {
        int64_t b = 0;
        if (d.off[r] < 0) continue;
        if (!role_shape(p, d, r, &b)) { fail("role " + std::to_string(r) + " leading dimension below its columns", it); continue; }
        if (d.off[r] < p->data_off || d.off[r] + b > ws) fail("role " + std::to_string(r) + " outside the workspace", it);
        // operand roles: 16-byte rows for the GEMMs' 16-byte loads; the dense
        // output U of a head block starts at row offset hr x cols, so it is
        // only element-aligned (its stores check alignment per access)
        if (r != R_U && (d.off[r] % 16 || (int64_t)d.ld[r] % 8))
          fail("role " + std::to_string(r) + " not 16-byte aligned", it);
        if (r == R_U && d.off[r] % p->mats[d.matrix].elem) fail("U not element-aligned", it);
        if (r != R_U) spans.push_back({d.off[r], d.off[r] + b, (int)pi, r});
      }
      // U aliases the X copy of its matrix that the last launch does not read
      const MatrixPlan &M = p->mats[d.matrix];
      int64_t ub = 0;
      if (role_shape(p, d, R_U, &ub)) {
        bool inside = false;
        for (int par = 0; par < 2; ++par) {
          const int64_t lo = p->data_off + M.orig_off[par];
          const int64_t hi = lo + M.desc.rows * M.ldc * M.elem;
          if (d.off[R_U] >= lo && d.off[R_U] + ub <= hi) inside = true;
        }
        if (!inside) fail("U outside the X copy it aliases", it);
      }
    }
    // X copies of one matrix are shared by its head blocks (disjoint row
    // ranges); all other buffers are private
    std::sort(spans.begin(), spans.end(), [](const Span &a, const Span &b) { return a.lo < b.lo; });
    for (size_t i = 1; i < spans.size(); ++i)
      if (spans[i].lo < spans[i - 1].hi)
        fail("buffers overlap: problem " + std::to_string(spans[i - 1].prob) + " role " +
                 std::to_string(spans[i - 1].role) + " and problem " + std::to_string(spans[i].prob) + " role " +
                 std::to_string(spans[i].role),
             it);
    // tile lists
    for (int g = 0; g < NGROUPS; ++g)
      for (int l = 0; l < NLISTS; ++l) {
        const int T = (l == TL_MM256 || l == TL_MN256) ? BIG_TILE : GEMM_TILE;
        const bool mn = (l == TL_MN128 || l == TL_MN256);
        for (const TileDev &t : W.tiles[g][l]) {
          if (t.prob < 0 || t.prob >= (int)W.probs.size()) { fail("tile of an unknown problem", it); continue; }
          const ProbDev &d = W.probs[t.prob];
          const int64_t N = mn ? d.n : d.m;
          if (t.tm < 0 || t.tn < 0 || (int64_t)t.tm * T >= d.m || (int64_t)t.tn * T >= N) fail("tile outside its problem", it);
          if (!mn && t.tm > t.tn) fail("lower-triangle tile in a symmetric list", it);
          if (T == BIG_TILE && d.m < BIG_TILE_MIN_M) fail("large tile on a small problem", it);
        }
      }
    // fused blocks (bf16, 64 <= m <= 128, at least one step): one entry each
    // in the fused group's list, X0 in both layouts and U allocated, U not
    // aliasing the parity-0 copy they read, no m x m buffer, and no tile in
    // any other list
    {
      std::vector<int> fused(W.probs.size(), 0), tiled(W.probs.size(), 0);
      for (const TileDev &t : W.tiles[PG_HEAD][TL_MN128]) {
        if (t.prob < 0 || t.prob >= (int)W.probs.size()) continue;
        ++fused[t.prob];
        if (t.tm != 0 || t.tn != 0) fail("fused entry with a tile position", it);
      }
      if (!W.tiles[PG_HEAD][TL_MM128].empty() || !W.tiles[PG_HEAD][TL_MM256].empty() ||
          !W.tiles[PG_HEAD][TL_MN256].empty())
        fail("fused group with tile lists", it);
      for (int g = 0; g < NGROUPS; ++g)
        for (int l = 0; l < NLISTS; ++l)
          if (g != PG_HEAD)
            for (const TileDev &t : W.tiles[g][l])
              if (t.prob >= 0 && t.prob < (int)W.probs.size()) ++tiled[t.prob];
      for (size_t pi = 0; pi < W.probs.size(); ++pi) {
        const ProbDev &d = W.probs[pi];
        const MatrixPlan &M = p->mats[d.matrix];
        const bool want = p->opt.ns_steps > 0 && !M.ops32 && d.m <= HEAD_MAX_M;
        if (want != (fused[pi] > 0)) fail("fused group membership", it);
        if (fused[pi] > 1) fail("fused block listed twice", it);
        if (fused[pi] && tiled[pi]) fail("fused block also tiled", it);
        if (!fused[pi] && !tiled[pi]) fail("block in no list", it);
        if (fused[pi]) {
          if (d.m < BF16_MIN_M) fail("fused block below the bf16 minimum", it);
          if (d.off[R_XR0] < 0 || d.off[R_XC0] < 0 || d.off[R_U] < 0) fail("fused block without X0 or U", it);
          for (int r = R_MA; r <= R_QB; ++r)
            if (d.off[r] >= 0) fail("fused block with an m x m buffer", it);
          const int64_t lo0 = p->data_off + M.orig_off[0], hi0 = lo0 + M.desc.rows * M.ldc * M.elem;
          if (d.off[R_U] >= lo0 && d.off[R_U] < hi0) fail("fused block's U aliases the copy it reads", it);
        }
      }
    }
    // persistent queues: for every large-tile group, exactly the tiles of
    // every launch of its schedule, each problem's items in one queue with
    // its launches in order (an item then waits only on earlier items of
    // its own queue), the tile counts and launch prefixes the kernel's
    // dependency test reads, zero counters, and an LPT spread of the work
    {
      const int np = (int)W.probs.size();
      const bool persistent = p->opt.schedule == MUON_SCHED_PERSISTENT;
      for (int g = 0; g < NGROUPS; ++g) {
        const std::vector<TileDev> &Q = W.pq[g];
        const std::vector<Launch> &S = p->schedule[g];
        const std::vector<TileDev> &MM = W.tiles[g][TL_MM256], &MN = W.tiles[g][TL_MN256];
        const bool want = persistent && g >= PG_BF16_BIG && !MN.empty() && p->opt.ns_steps > 0;
        if (want != !Q.empty()) { fail("persistent queue presence", it); continue; }
        if (Q.empty()) continue;
        ++g_queued;
        if (W.pq_off[g][0] != 0 || W.pq_off[g][PQ_XCDS] != (int32_t)Q.size()) fail("queue bounds", it);
        for (int x = 0; x < PQ_XCDS; ++x)
          if (W.pq_off[g][x] > W.pq_off[g][x + 1]) fail("queue bounds out of order", it);
        if (!in_tables(W.off_pq[g], (int64_t)(Q.size() * sizeof(TileDev))) ||
            !in_tables(W.off_pl[g], (int64_t)(W.pl[g].size() * sizeof(PLaunch))) ||
            !in_tables(W.off_pcnt[g], (int64_t)(PQ_XCDS + np) * PQ_PAD * 4) ||
            !in_tables(W.off_pntl, (int64_t)W.pntl.size() * 4))
          fail("a persistent table leaves the table region", it);
        for (int64_t b = 0; b < (int64_t)(PQ_XCDS + np) * PQ_PAD * 4; ++b)
          if (p->host_tables[W.off_pcnt[g] + b] != 0) { fail("persistent counters not zero", it); break; }
        // the items against the schedule's launches over the tile lists
        std::vector<std::array<int32_t, 4>> want_items, got_items;
        for (size_t k = 0; k < S.size(); ++k)
          for (const TileDev &t : (S[k].mn ? MN : MM)) want_items.push_back({t.prob, (int32_t)k, t.tm, t.tn});
        std::vector<int> xcd_of(np, -1), last_k(np, -1);
        std::vector<double> load(PQ_XCDS, 0.0);
        double biggest = 0.0;
        for (int x = 0; x < PQ_XCDS; ++x)
          for (int32_t i = W.pq_off[g][x]; i < W.pq_off[g][x + 1]; ++i) {
            const int32_t pr = Q[i].prob & PQ_PROB_MASK, k = (int32_t)((uint32_t)Q[i].prob >> PQ_LAUNCH_SHIFT);
            got_items.push_back({pr, k, Q[i].tm, Q[i].tn});
            if (pr < 0 || pr >= np || k >= (int32_t)S.size()) { fail("queue item out of range", it); continue; }
            if (xcd_of[pr] < 0) {
              xcd_of[pr] = x;
              const double f = p->probs[W.problems[pr]].flops;
              load[x] += f;
              biggest = std::max(biggest, f);
            }
            if (xcd_of[pr] != x) fail("a problem in two queues", it);
            if (k < last_k[pr]) fail("a problem's launches out of order in its queue", it);
            last_k[pr] = k;
          }
        std::sort(want_items.begin(), want_items.end());
        std::sort(got_items.begin(), got_items.end());
        if (want_items != got_items) fail("queue items differ from the schedule's tiles", it);
        const auto mm = std::minmax_element(load.begin(), load.end());
        if (*mm.second - *mm.first > biggest * (1 + 1e-9)) fail("queues not balanced as LPT", it);
        // tile counts per problem and the launch prefixes
        std::vector<int32_t> nmm(np, 0), nmn(np, 0);
        for (const TileDev &t : MM) ++nmm[t.prob];
        for (const TileDev &t : MN) ++nmn[t.prob];
        for (int pr = 0; pr < np; ++pr)
          if (nmn[pr] && (W.pntl[2 * pr] != nmm[pr] || W.pntl[2 * pr + 1] != nmn[pr])) fail("problem tile counts", it);
        if (W.pl[g].size() != S.size()) { fail("launch table size", it); continue; }
        int32_t cm = 0, cn = 0;
        for (size_t k = 0; k < S.size(); ++k) {
          if (W.pl[g][k].mm_before != cm || W.pl[g][k].mn_before != cn) fail("launch prefixes", it);
          if (std::memcmp(&W.pl[g][k].r, &S[k].r, sizeof(GemmRecipe)) != 0) fail("launch recipe", it);
          (S[k].mn ? cn : cm) += 1;
        }
      }
    }
    // K1 entries
    int32_t k1t = 0;
    for (const K1Prob &k : W.k1) {
      if (k.tile0 != k1t) fail("K1 tile prefix", it);
      if (k.ntiles != cdiv(k.hr, K1_TILE) * cdiv(k.cols, K1_TILE)) fail("K1 tile count", it);
      k1t += k.ntiles;
      const int64_t e = k.xbf16 ? 2 : 4;
      if (k.orig_off < p->data_off || k.orig_off + ((int64_t)(k.hr - 1) * k.orig_ld + k.cols) * e > ws)
        fail("K1 original copy outside the workspace", it);
      if (k.trans_off < p->data_off || k.trans_off + ((k.cols - 1) * k.trans_ld + k.hr) * e > ws)
        fail("K1 transposed copy outside the workspace", it);
    }
    if (k1t != W.k1_tiles) fail("K1 tile total", it);
    // writeback runs
    int64_t ch = 0;
    for (size_t j = 0; j < W.runs.size(); ++j) {
      const K3Run &r = W.runs[j];
      const muon_run &s = W.run_src[j];
      const muon_matrix &D = p->mats[s.matrix].desc;
      if (r.first != s.first || r.length != s.length || r.chunk0 != ch) fail("K3 run mismatch", it);
      if (s.first < 0 || s.length < 1 || s.first + s.length > D.rows * D.cols) fail("run outside its matrix", it);
      if (s.partition < 0 || s.partition >= p->layout.num_partitions || s.offset < 0 || s.offset + s.length > P)
        fail("run outside its partition", it);
      ch += cdiv(s.length, K3_CHUNK);
    }
    if (ch != W.k3_chunks || W.k3_base != nparts) fail("K3 chunk count", it);
    nparts += ch;
  }
  if (nparts != p->nparts_n) fail("norm partial count", it);
  if (p->nparts_off + p->nparts_n * 4 > p->nc_off) fail("norm partials overlap", it);
}

int64_t pick_side(std::mt19937_64 &rng) {
  const int k = (int)(rng() % 10);
  if (k < 4) return 1 + (int64_t)(rng() % 40);          // tiny, ragged
  if (k < 8) return 40 + (int64_t)(rng() % 700);        // across the 128 / 256 tiles
  if (k < 9) return 1024 + 64 * (int64_t)(rng() % 8);   // large-tile multiples
  return 2048 + (int64_t)(rng() % 700);                 // the lean Gram class
}

}  // namespace

int main(int argc, char **argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const uint64_t iters = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 200;
  std::mt19937_64 rng(seed);
  uint64_t planned = 0;
  for (uint64_t it = 0; it < iters; ++it) {
    const int n = 1 + (int)(rng() % 7);
    std::vector<muon_matrix> mats(n);
    int64_t total = 0;
    const bool interior = rng() & 1;
    for (int i = 0; i < n; ++i) {
      muon_matrix &M = mats[i];
      M.rows = pick_side(rng);
      M.cols = pick_side(rng);
      if (M.rows * M.cols > 6000000) M.cols = std::max<int64_t>(1, 6000000 / M.rows);
      M.num_heads = 0;
      if (rng() % 3 == 0) {
        const int h = 1 + (int)(rng() % 8);
        if (M.rows % h == 0) M.num_heads = h;
      }
      M.reserved = 0;
      if (interior) total = (total + 15) / 16 * 16;
      M.flat_offset = total;
      total += M.rows * M.cols;
    }
    muon_options o;
    muon_default_options(&o);
    o.method = (rng() & 1) ? MUON_NS_GRAM : MUON_NS_STANDARD;
    o.precision = (rng() % 4) ? MUON_PREC_BF16 : MUON_PREC_FP32;
    o.ns_steps = (int)(rng() % 6);
    o.grad_dtype = (rng() & 1) ? MUON_DT_BF16 : MUON_DT_FP32;
    o.schedule = (rng() & 1) ? MUON_SCHED_PERSISTENT : MUON_SCHED_LAUNCHES;
    const int R = 1 + (int)(rng() % 5);
    muon_layout lay;
    lay.num_partitions = R;
    lay.partition_numel = std::max<int64_t>(1, (total + R * 16 - 1) / (R * 16) * 16);
    lay.reserved = 0;
    muon_plan *p = nullptr;
    muon_status st = muon_plan_create(&p, mats.data(), n, &o, &lay);
    if (st != MUON_OK) { fail(std::string("valid group refused: ") + muon_last_error(), it); continue; }
    // a cap of a fraction of the uncapped workspace cuts the group into waves
    if (rng() & 1) {
      const uint64_t cap = (uint64_t)p->ws_bytes / (2 + rng() % 6);
      delete p;
      o.max_inflight_bytes = cap;
      st = muon_plan_create(&p, mats.data(), n, &o, &lay);
      if (st != MUON_OK) { fail(std::string("capped group refused: ") + muon_last_error(), it); continue; }
    }
    check_plan(p, it);
    // the introspection calls with a short output array
    int32_t count = -1;
    muon_run one_run;
    if (muon_plan_runs(p, 0, &one_run, 1, &count) != MUON_OK || count < 1) fail("muon_plan_runs", it);
    muon_problem_info one;
    if (muon_plan_problems(p, &one, 1, &count) != MUON_OK || count < n) fail("muon_plan_problems", it);
    ++planned;
    delete p;  // host-only: the plan holds no HIP resource until a step runs
  }
  // refused groups: each returns its status and leaves *out NULL
  {
    muon_options o;
    muon_default_options(&o);
    muon_layout lay{64, 1, 0};
    struct Bad { muon_matrix m[2]; int n; muon_status want; } bad[] = {
        {{{0, 4, 0, 0, 0}}, 1, MUON_ERR_INVALID_ARG},
        {{{6, 4, 4, 0, 0}}, 1, MUON_ERR_UNSUPPORTED},
        {{{4, 4, -1, 0, 0}}, 1, MUON_ERR_INVALID_ARG},
        {{{4, 4, 0, 0, 0}, {4, 4, 0, 0, 8}}, 2, MUON_ERR_LAYOUT},
        {{{8, 9, 0, 0, 0}}, 1, MUON_ERR_LAYOUT},
        {{{4, 4, 0, 1, 0}}, 1, MUON_ERR_INVALID_ARG},
    };
    for (const Bad &b : bad) {
      muon_plan *p = reinterpret_cast<muon_plan *>(&lay);
      if (muon_plan_create(&p, b.m, b.n, &o, &lay) != b.want || p != nullptr) fail("an invalid group", 0);
    }
  }
  if (g_fail) {
    std::fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  std::printf("plan invariants ok: %llu plans, %llu persistent queues\n", (unsigned long long)planned,
              (unsigned long long)g_queued);
  return 0;
}
