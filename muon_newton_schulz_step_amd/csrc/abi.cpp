// C ABI entry points that touch the device: muon_step, muon_accumulate,
// muon_scatter, muon_check_finite, muon_apply_update, muon_plan_destroy, and
// the pieces of a step (check, table patch, launches, counters) that every
// entry point running a step shares.
// All argument checks run before anything is enqueued.  Launch tables are
// uploaded into the head of the caller's workspace from pinned host staging
// (two slots, each guarded by an event, so the host never overwrites a
// buffer the copy engine still reads).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "elem.hpp"
#include "muon.h"
#include "plan.hpp"

using namespace muon;

namespace {

using Range = AddrRange;

muon_status check_alias(std::vector<Range> &rs) {
  std::sort(rs.begin(), rs.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
  for (size_t i = 1; i < rs.size(); ++i) {
    if (rs[i].lo < rs[i - 1].hi) {
      set_error(std::string("buffers overlap: ") + rs[i - 1].what + "[" + std::to_string(rs[i - 1].index) + "] and " +
                rs[i].what + "[" + std::to_string(rs[i].index) + "]");
      return MUON_ERR_ALIAS;
    }
  }
  return MUON_OK;
}

muon_status hip_fail(hipError_t e, const char *where) {
  set_error(std::string(where) + ": " + hipGetErrorString(e));
  return MUON_ERR_HIP;
}

muon_status ensure_staging(muon_plan *p, size_t bytes) {
  if (p->staging_bytes >= bytes && p->staging[0]) return MUON_OK;
  for (int s = 0; s < 2; ++s) {
    if (p->event_live[s]) {
      hipError_t e = hipEventSynchronize((hipEvent_t)p->events[s]);
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      p->event_live[s] = false;
    }
    if (p->staging[s]) {
      (void)hipHostFree(p->staging[s]);
      p->staging[s] = nullptr;
    }
  }
  p->staging_bytes = 0;
  const size_t want = std::max<size_t>(bytes, 4096);
  for (int s = 0; s < 2; ++s) {
    hipError_t e = hipHostMalloc(&p->staging[s], want, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc (table staging)");
    if (!p->events[s]) {
      hipEvent_t ev;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
      p->events[s] = ev;
    }
  }
  p->staging_bytes = want;
  return MUON_OK;
}

// Take the next staging slot once the copy that last used it has finished.
muon_status acquire_slot(muon_plan *p, size_t bytes, char **host, int *slot) {
  muon_status st = ensure_staging(p, bytes);
  if (st != MUON_OK) return st;
  const int s = p->slot;
  p->slot ^= 1;
  if (p->event_live[s]) {
    hipError_t e = hipEventSynchronize((hipEvent_t)p->events[s]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    p->event_live[s] = false;
  }
  *host = static_cast<char *>(p->staging[s]);
  *slot = s;
  return MUON_OK;
}

muon_status upload(muon_plan *p, int slot, void *dst, size_t bytes, hipStream_t s) {
  if (bytes == 0) return MUON_OK;
  hipError_t e = hipMemcpyAsync(dst, p->staging[slot], bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (tables)");
  e = hipEventRecord((hipEvent_t)p->events[slot], s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  p->event_live[slot] = true;
  return MUON_OK;
}

size_t dtype_size(int32_t dt) { return dt == MUON_DT_BF16 ? 2 : 4; }

muon_status check_ws(const muon_plan *p, void *ws, size_t ws_bytes, size_t need) {
  if (!ws) { set_error("workspace is NULL"); return MUON_ERR_WORKSPACE; }
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) { set_error("workspace must be 256-byte aligned"); return MUON_ERR_WORKSPACE; }
  if (ws_bytes < need) {
    set_error("workspace too small: " + std::to_string(ws_bytes) + " < " + std::to_string(need));
    return MUON_ERR_WORKSPACE;
  }
  (void)p;
  return MUON_OK;
}

}  // namespace

namespace muon {

muon_status step_check(muon_plan *p, const void *const *grads, float *const *momenta, float *const *partitions,
                       const int32_t *skip_flag, float grad_scale, void *ws, size_t ws_bytes) {
  if (!p || !grads || !momenta || !partitions) { set_error("muon_step: NULL argument"); return MUON_ERR_INVALID_ARG; }
  if (!std::isfinite(grad_scale)) { set_error("muon_step: grad_scale is not finite"); return MUON_ERR_INVALID_ARG; }
  const int32_t nmat = (int32_t)p->mats.size();
  const int32_t R = p->layout.num_partitions;
  const size_t gsz = dtype_size(p->opt.grad_dtype);
  std::vector<AddrRange> &rs = p->ranges;  // capacity reserved at plan creation
  rs.clear();
  for (int32_t i = 0; i < nmat; ++i) {
    if (!grads[i] || !momenta[i]) { set_error("muon_step: NULL grads/momenta entry " + std::to_string(i)); return MUON_ERR_INVALID_ARG; }
    const uintptr_t n = (uintptr_t)(p->mats[i].desc.rows * p->mats[i].desc.cols);
    rs.push_back({(uintptr_t)grads[i], (uintptr_t)grads[i] + n * gsz, "grads", i});
    rs.push_back({(uintptr_t)momenta[i], (uintptr_t)momenta[i] + n * 4, "momenta", i});
  }
  for (int32_t r = 0; r < R; ++r) {
    if (!partitions[r]) { set_error("muon_step: NULL partition " + std::to_string(r)); return MUON_ERR_INVALID_ARG; }
    rs.push_back({(uintptr_t)partitions[r], (uintptr_t)partitions[r] + (uintptr_t)p->layout.partition_numel * 4,
                  "partitions", r});
  }
  muon_status st = check_ws(p, ws, ws_bytes, (size_t)p->ws_bytes);
  if (st != MUON_OK) return st;
  rs.push_back({(uintptr_t)ws, (uintptr_t)ws + ws_bytes, "workspace", 0});
  if (skip_flag) rs.push_back({(uintptr_t)skip_flag, (uintptr_t)skip_flag + 4, "skip_flag", 0});
  return check_alias(rs);
}

void step_patch(const muon_plan *p, char *h, const void *const *grads, float *const *momenta,
                float *const *partitions, char *wsb) {
  std::memcpy(h, p->host_tables.data(), p->host_tables.size());
  for (const WavePlan &W : p->waves) {
    K1Prob *k1 = reinterpret_cast<K1Prob *>(h + W.off_k1);
    for (size_t j = 0; j < W.k1.size(); ++j) {
      k1[j].grad = grads[W.k1_matrix[j]];
      k1[j].mom = momenta[W.k1_matrix[j]];
    }
    K3Run *runs = reinterpret_cast<K3Run *>(h + W.off_runs);
    for (size_t j = 0; j < W.runs.size(); ++j) {
      const muon_run &r = W.run_src[j];
      runs[j].src = wsb + p->mats[r.matrix].u_off;
      runs[j].dst = partitions[r.partition] + r.offset;
    }
  }
}

// The plan's second stream and its fork / join events, created once.
static muon_status ensure_side(muon_plan *p) {
  if (p->side_stream) return MUON_OK;
  hipEvent_t f = nullptr, j = nullptr;
  hipStream_t s2 = nullptr;
  hipError_t e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&s2, hipStreamNonBlocking);
  if (e != hipSuccess) {
    if (f) (void)hipEventDestroy(f);
    if (j) (void)hipEventDestroy(j);
    return hip_fail(e, "second stream");
  }
  p->fork_ev = f;
  p->join_ev = j;
  p->side_stream = s2;
  return MUON_OK;
}

// The persistent schedule assumes 8 XCDs of 32 CUs, one workgroup each,
// with workgroup i on XCD i mod 8 (true of MI355X with all its CUs in one
// partition); on any other device the step falls back to the launches.
static bool persistent_fits() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  return cus == PQ_XCDS * 32;
}

muon_status step_launch(muon_plan *p, const int32_t *skip_flag, float grad_scale, char *wsb, void *stream,
                        bool timed, bool side) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  timed = timed && p->timing;
  if (timed) {
    const size_t need = 4 * p->waves.size();
    while (p->phase_events.size() < need) {
      hipEvent_t ev;
      hipError_t e = hipEventCreate(&ev);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate (timing)");
      p->phase_events.push_back(ev);
    }
  }
  auto mark = [&](size_t w, int k) -> hipError_t {
    if (!timed) return hipSuccess;
    return hipEventRecord((hipEvent_t)p->phase_events[4 * w + k], s);
  };
  int32_t ns_launches = 0;
  size_t wi = 0;
  const bool gbf16 = p->opt.grad_dtype == MUON_DT_BF16;
  float *partials = reinterpret_cast<float *>(wsb + p->partials_off);
  float *scales = reinterpret_cast<float *>(wsb + p->scales_off);
  float *nparts = reinterpret_cast<float *>(wsb + p->nparts_off);
  hipError_t e;
  for (const WavePlan &W : p->waves) {
    const int np = (int)W.probs.size();
    const K1Prob *k1 = reinterpret_cast<const K1Prob *>(wsb + W.off_k1);
    const ProbDev *probs = reinterpret_cast<const ProbDev *>(wsb + W.off_prob);
    const K3Run *runs = reinterpret_cast<const K3Run *>(wsb + W.off_runs);
    if ((e = mark(wi, 0)) != hipSuccess) return hip_fail(e, "hipEventRecord (timing)");
    if ((e = launch_k1(k1, np, W.k1_tiles, wsb, partials, p->opt.beta, p->opt.nesterov, grad_scale, skip_flag, gbf16,
                       s)) != hipSuccess)
      return hip_fail(e, "K1 launch");
    if ((e = launch_kn(k1, np, partials, scales, p->opt.eps, skip_flag, s)) != hipSuccess)
      return hip_fail(e, "norm launch");
    if ((e = mark(wi, 1)) != hipSuccess) return hip_fail(e, "hipEventRecord (timing)");
    if (p->opt.ns_steps == 0) {
      if ((e = launch_kc(probs, k1, np, wsb, scales, skip_flag, s)) != hipSuccess) return hip_fail(e, "copy launch");
    } else {
      // Large bf16 problems first (the bulk of the work), then small bf16
      // ones, then fp32-operand ones.  When a wave holds both large-tile and
      // small-block groups, the small ones run on the second stream: their
      // launches are short, mostly bound by HBM, and would otherwise wait
      // for every large-tile launch; the groups share no buffer.
      bool big_any = false, small_any = false;
      for (int grp = 0; grp < NGROUPS; ++grp) {
        if (W.tiles[grp][TL_MN128].empty()) continue;
        (grp >= PG_BF16_BIG ? big_any : small_any) = true;
      }
      const bool fork = side && big_any && small_any;
      hipStream_t s2 = s;
      if (fork) {
        muon_status st = ensure_side(p);
        if (st != MUON_OK) return st;
        s2 = static_cast<hipStream_t>(p->side_stream);
        if ((e = hipEventRecord((hipEvent_t)p->fork_ev, s)) != hipSuccess) return hip_fail(e, "hipEventRecord (fork)");
        if ((e = hipStreamWaitEvent(s2, (hipEvent_t)p->fork_ev, 0)) != hipSuccess)
          return hip_fail(e, "hipStreamWaitEvent (fork)");
      }
      const bool persist = p->opt.schedule == MUON_SCHED_PERSISTENT && persistent_fits();
      for (int grp = NGROUPS - 1; grp >= PG_F32; --grp) {
        if (W.tiles[grp][TL_MN128].empty()) continue;
        const std::vector<Launch> &sched = p->schedule[grp];
        hipStream_t sg = grp >= PG_BF16_BIG ? s : s2;
        if (persist && !W.pq[grp].empty()) {
          // every product of every problem of the group in one launch
          PersistArgs pa;
          pa.probs = probs; pa.ws = wsb; pa.scales = scales; pa.skip = skip_flag;
          pa.launches = reinterpret_cast<const PLaunch *>(wsb + W.off_pl[grp]);
          pa.items = reinterpret_cast<const TileDev *>(wsb + W.off_pq[grp]);
          pa.ntl = reinterpret_cast<const int32_t *>(wsb + W.off_pntl);
          pa.counters = reinterpret_cast<int32_t *>(wsb + W.off_pcnt[grp]);
          for (int x = 0; x <= PQ_XCDS; ++x) pa.qoff[x] = W.pq_off[grp][x];
          bool split = false;
          for (const Launch &L : sched) split = split || L.r.nseg > 1 || (L.r.flags & (GF_SPLIT_OUT | GF_D_SPLIT));
          if ((e = launch_persist(pa, split, sg)) != hipSuccess) return hip_fail(e, "Newton-Schulz launch (persistent)");
          ++ns_launches;
          continue;
        }
        if (grp == PG_HEAD) {
          // one workgroup per block runs its whole iteration
          const TileDev *tl = reinterpret_cast<const TileDev *>(wsb + W.off_tiles[grp][TL_MN128]);
          HeadArgs ha{probs, tl, wsb, scales, skip_flag, p->opt.a, p->opt.b, p->opt.c, p->opt.ns_steps,
                      p->opt.method == MUON_NS_STANDARD ? 1 : 0};
          if ((e = launch_head(ha, (int)W.tiles[grp][TL_MN128].size(), sg)) != hipSuccess)
            return hip_fail(e, "Newton-Schulz launch (fused blocks)");
          ++ns_launches;
          continue;
        }
        for (const Launch &L : sched) {
          const bool big = grp >= PG_BF16_BIG && L.kind == Launch::GEMM_OP;
          const int list = big ? (L.mn ? TL_MN256 : TL_MM256) : (L.mn ? TL_MN128 : TL_MM128);
          const TileDev *tl = reinterpret_cast<const TileDev *>(wsb + W.off_tiles[grp][list]);
          const int nt = (int)W.tiles[grp][list].size();
          GemmArgs a{probs, tl, wsb, scales, L.r, skip_flag};
          e = big ? launch_gemm256(a, nt, sg) : launch_gemm(L.kind == Launch::GEMM_OP, a, nt, sg);
          if (e != hipSuccess) return hip_fail(e, "Newton-Schulz launch");
          ++ns_launches;
        }
      }
      if (fork) {
        if ((e = hipEventRecord((hipEvent_t)p->join_ev, s2)) != hipSuccess) return hip_fail(e, "hipEventRecord (join)");
        if ((e = hipStreamWaitEvent(s, (hipEvent_t)p->join_ev, 0)) != hipSuccess)
          return hip_fail(e, "hipStreamWaitEvent (join)");
      }
    }
    if ((e = mark(wi, 2)) != hipSuccess) return hip_fail(e, "hipEventRecord (timing)");
    if ((e = launch_k3(runs, (int)W.runs.size(), W.k3_chunks, skip_flag, nparts, W.k3_base, s)) != hipSuccess)
      return hip_fail(e, "K3 launch");
    if ((e = mark(wi, 3)) != hipSuccess) return hip_fail(e, "hipEventRecord (timing)");
    ++wi;
  }
  if (timed) {
    p->timed_step = true;
    p->timed_launches = ns_launches;
  }
  return MUON_OK;
}

void step_count(muon_plan *p, const int32_t *skip_flag, const void *ws) {
  p->stats.steps += 1;
  p->stats.ns_invocations += (uint64_t)p->mats.size();
  if (skip_flag) p->stats.flagged_steps += 1;
  p->norm_ws = ws;
}

}  // namespace muon

extern "C" {

muon_status muon_step(muon_plan *p, const void *const *grads, float *const *momenta, float *const *partitions, void *ws,
                      size_t ws_bytes, void *stream) {
  return muon_step_ex(p, grads, momenta, partitions, nullptr, 1.0f, ws, ws_bytes, stream);
}

muon_status muon_step_ex(muon_plan *p, const void *const *grads, float *const *momenta, float *const *partitions,
                         const int32_t *skip_flag, float grad_scale, void *ws, size_t ws_bytes, void *stream) {
  muon_status st = step_check(p, grads, momenta, partitions, skip_flag, grad_scale, ws, ws_bytes);
  if (st != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *h = nullptr;
  int slot = 0;
  if ((st = acquire_slot(p, p->host_tables.size(), &h, &slot)) != MUON_OK) return st;
  char *wsb = static_cast<char *>(ws);
  step_patch(p, h, grads, momenta, partitions, wsb);
  if ((st = upload(p, slot, ws, p->host_tables.size(), s)) != MUON_OK) return st;
  if ((st = step_launch(p, skip_flag, grad_scale, wsb, stream, true, true)) != MUON_OK) return st;
  step_count(p, skip_flag, ws);
  return MUON_OK;
}

muon_status muon_accumulate(muon_plan *p, float *const *acc, const void *const *grad_mb, int32_t mb_dtype,
                            int32_t first, void *ws, size_t ws_bytes, void *stream) {
  if (!p || !acc || !grad_mb) { set_error("muon_accumulate: NULL argument"); return MUON_ERR_INVALID_ARG; }
  if (mb_dtype != MUON_DT_FP32 && mb_dtype != MUON_DT_BF16) { set_error("muon_accumulate: unknown dtype"); return MUON_ERR_INVALID_ARG; }
  const int32_t nmat = (int32_t)p->mats.size();
  const size_t gsz = dtype_size(mb_dtype);
  std::vector<Range> rs;
  std::vector<K0Mat> tab(nmat);
  int64_t ch = 0;
  for (int32_t i = 0; i < nmat; ++i) {
    if (!acc[i] || !grad_mb[i]) { set_error("muon_accumulate: NULL entry " + std::to_string(i)); return MUON_ERR_INVALID_ARG; }
    const int64_t n = p->mats[i].desc.rows * p->mats[i].desc.cols;
    rs.push_back({(uintptr_t)acc[i], (uintptr_t)acc[i] + (uintptr_t)n * 4, "acc", i});
    rs.push_back({(uintptr_t)grad_mb[i], (uintptr_t)grad_mb[i] + (uintptr_t)n * gsz, "grad_mb", i});
    tab[i] = K0Mat{acc[i], grad_mb[i], n, ch};
    ch += (n + K0_CHUNK - 1) / K0_CHUNK;
  }
  const size_t tb = tab.size() * sizeof(K0Mat);
  muon_status st = check_ws(p, ws, ws_bytes, tb);
  if (st != MUON_OK) return st;
  rs.push_back({(uintptr_t)ws, (uintptr_t)ws + ws_bytes, "workspace", 0});
  if ((st = check_alias(rs)) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *h = nullptr;
  int slot = 0;
  if ((st = acquire_slot(p, std::max<size_t>(tb, p->host_tables.size()), &h, &slot)) != MUON_OK) return st;
  std::memcpy(h, tab.data(), tb);
  if ((st = upload(p, slot, ws, tb, s)) != MUON_OK) return st;
  hipError_t e = launch_k0(static_cast<const K0Mat *>(ws), nmat, ch, mb_dtype == MUON_DT_BF16, first ? 1 : 0, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  p->stats.accumulations += 1;
  return MUON_OK;
}

muon_status muon_scatter(muon_plan *p, const void *const *updates, int32_t dtype, float *const *partitions, void *ws,
                         size_t ws_bytes, void *stream) {
  if (!p || !updates || !partitions) { set_error("muon_scatter: NULL argument"); return MUON_ERR_INVALID_ARG; }
  if (dtype != MUON_DT_FP32 && dtype != MUON_DT_BF16) { set_error("muon_scatter: unknown dtype"); return MUON_ERR_INVALID_ARG; }
  const int32_t nmat = (int32_t)p->mats.size();
  const int32_t R = p->layout.num_partitions;
  const size_t usz = dtype_size(dtype);
  std::vector<Range> rs;
  for (int32_t i = 0; i < nmat; ++i) {
    if (!updates[i]) { set_error("muon_scatter: NULL update " + std::to_string(i)); return MUON_ERR_INVALID_ARG; }
    const int64_t n = p->mats[i].desc.rows * p->mats[i].desc.cols;
    rs.push_back({(uintptr_t)updates[i], (uintptr_t)updates[i] + (uintptr_t)n * usz, "updates", i});
  }
  for (int32_t r = 0; r < R; ++r) {
    if (!partitions[r]) { set_error("muon_scatter: NULL partition " + std::to_string(r)); return MUON_ERR_INVALID_ARG; }
    rs.push_back({(uintptr_t)partitions[r], (uintptr_t)partitions[r] + (uintptr_t)p->layout.partition_numel * 4,
                  "partitions", r});
  }
  std::vector<K3Run> tab;
  int64_t ch = 0;
  for (int32_t i = 0; i < nmat; ++i) {
    for (const muon_run &r : p->mats[i].runs) {
      K3Run k;
      std::memset(&k, 0, sizeof(k));
      k.src = updates[i];
      k.dst = partitions[r.partition] + r.offset;
      k.first = r.first;
      k.length = r.length;
      k.chunk0 = ch;
      k.scale = p->mats[i].scale;
      k.src_bf16 = dtype == MUON_DT_BF16 ? 1 : 0;
      ch += (r.length + K3_CHUNK - 1) / K3_CHUNK;
      tab.push_back(k);
    }
  }
  const size_t tb = tab.size() * sizeof(K3Run);
  muon_status st = check_ws(p, ws, ws_bytes, tb);
  if (st != MUON_OK) return st;
  rs.push_back({(uintptr_t)ws, (uintptr_t)ws + ws_bytes, "workspace", 0});
  if ((st = check_alias(rs)) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *h = nullptr;
  int slot = 0;
  if ((st = acquire_slot(p, std::max<size_t>(tb, p->host_tables.size()), &h, &slot)) != MUON_OK) return st;
  std::memcpy(h, tab.data(), tb);
  if ((st = upload(p, slot, ws, tb, s)) != MUON_OK) return st;
  hipError_t e = launch_k3(static_cast<const K3Run *>(ws), (int)tab.size(), ch, nullptr, nullptr, 0, s);
  if (e != hipSuccess) return hip_fail(e, "scatter launch");
  return MUON_OK;
}

muon_status muon_check_finite(muon_plan *p, const void *const *grads, int32_t dtype, int32_t *flag, void *ws,
                              size_t ws_bytes, void *stream) {
  if (!p || !grads || !flag) { set_error("muon_check_finite: NULL argument"); return MUON_ERR_INVALID_ARG; }
  if (dtype != MUON_DT_FP32 && dtype != MUON_DT_BF16) { set_error("muon_check_finite: unknown dtype"); return MUON_ERR_INVALID_ARG; }
  const int32_t nmat = (int32_t)p->mats.size();
  const size_t gsz = dtype_size(dtype);
  std::vector<Range> rs;
  std::vector<K0Mat> tab(nmat);
  int64_t ch = 0;
  for (int32_t i = 0; i < nmat; ++i) {
    if (!grads[i]) { set_error("muon_check_finite: NULL grads entry " + std::to_string(i)); return MUON_ERR_INVALID_ARG; }
    const int64_t n = p->mats[i].desc.rows * p->mats[i].desc.cols;
    rs.push_back({(uintptr_t)grads[i], (uintptr_t)grads[i] + (uintptr_t)n * gsz, "grads", i});
    tab[i] = K0Mat{nullptr, grads[i], n, ch};
    ch += (n + K0_CHUNK - 1) / K0_CHUNK;
  }
  const size_t tb = tab.size() * sizeof(K0Mat);
  muon_status st = check_ws(p, ws, ws_bytes, tb);
  if (st != MUON_OK) return st;
  rs.push_back({(uintptr_t)ws, (uintptr_t)ws + ws_bytes, "workspace", 0});
  rs.push_back({(uintptr_t)flag, (uintptr_t)flag + 4, "flag", 0});
  if ((st = check_alias(rs)) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *h = nullptr;
  int slot = 0;
  if ((st = acquire_slot(p, std::max<size_t>(tb, p->host_tables.size()), &h, &slot)) != MUON_OK) return st;
  std::memcpy(h, tab.data(), tb);
  if ((st = upload(p, slot, ws, tb, s)) != MUON_OK) return st;
  hipError_t e = launch_finite(static_cast<const K0Mat *>(ws), nmat, ch, dtype == MUON_DT_BF16, flag, s);
  if (e != hipSuccess) return hip_fail(e, "finite-check launch");
  return MUON_OK;
}

muon_status muon_apply_update(muon_plan *p, float *const *params, const float *const *partitions, float lr,
                              float weight_decay, float max_norm, const int32_t *skip_flag, float *norm_clip_out,
                              void *ws, size_t ws_bytes, void *stream) {
  if (!p || !params || !partitions) { set_error("muon_apply_update: NULL argument"); return MUON_ERR_INVALID_ARG; }
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(max_norm)) {
    set_error("muon_apply_update: lr, weight_decay and max_norm must be finite");
    return MUON_ERR_INVALID_ARG;
  }
  muon_status st = check_ws(p, ws, ws_bytes, (size_t)p->ws_bytes);
  if (st != MUON_OK) return st;
  if (p->norm_ws != ws) {
    set_error("muon_apply_update: no muon_step has run on this plan with this workspace");
    return MUON_ERR_INVALID_ARG;
  }
  const int32_t R = p->layout.num_partitions;
  const uintptr_t pb = (uintptr_t)p->layout.partition_numel * 4;
  std::vector<Range> rs;
  for (int32_t r = 0; r < R; ++r) {
    if (!params[r] || !partitions[r]) {
      set_error("muon_apply_update: NULL params/partitions entry " + std::to_string(r));
      return MUON_ERR_INVALID_ARG;
    }
    rs.push_back({(uintptr_t)params[r], (uintptr_t)params[r] + pb, "params", r});
    rs.push_back({(uintptr_t)partitions[r], (uintptr_t)partitions[r] + pb, "partitions", r});
  }
  rs.push_back({(uintptr_t)ws, (uintptr_t)ws + ws_bytes, "workspace", 0});
  if (skip_flag) rs.push_back({(uintptr_t)skip_flag, (uintptr_t)skip_flag + 4, "skip_flag", 0});
  if (norm_clip_out) rs.push_back({(uintptr_t)norm_clip_out, (uintptr_t)norm_clip_out + 8, "norm_clip_out", 0});
  if ((st = check_alias(rs)) != MUON_OK) return st;
  std::vector<KARun> tab;
  int64_t ch = 0;
  for (const auto &M : p->mats) {
    for (const muon_run &r : M.runs) {
      KARun k;
      k.param = params[r.partition] + r.offset;
      k.upd = partitions[r.partition] + r.offset;
      k.length = r.length;
      k.chunk0 = ch;
      ch += (r.length + KA_CHUNK - 1) / KA_CHUNK;
      tab.push_back(k);
    }
  }
  const size_t tb = tab.size() * sizeof(KARun);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *h = nullptr;
  int slot = 0;
  if ((st = acquire_slot(p, std::max<size_t>(tb, p->host_tables.size()), &h, &slot)) != MUON_OK) return st;
  std::memcpy(h, tab.data(), tb);
  if ((st = upload(p, slot, ws, tb, s)) != MUON_OK) return st;
  char *wsb = static_cast<char *>(ws);
  const float *nparts = reinterpret_cast<const float *>(wsb + p->nparts_off);
  float *nc = reinterpret_cast<float *>(wsb + p->nc_off);
  double *l1 = reinterpret_cast<double *>(wsb + p->nl1_off);
  hipError_t e = launch_norm_clip(nparts, p->nparts_n, l1, max_norm, nc, norm_clip_out, skip_flag, s);
  if (e != hipSuccess) return hip_fail(e, "norm launch");
  e = launch_apply(static_cast<const KARun *>(ws), (int)tab.size(), ch, nc, lr, weight_decay, skip_flag, s);
  if (e != hipSuccess) return hip_fail(e, "apply launch");
  return MUON_OK;
}

muon_status muon_plan_set_timing(muon_plan *p, int32_t enable) {
  if (!p) { set_error("muon_plan_set_timing: NULL plan"); return MUON_ERR_INVALID_ARG; }
  p->timing = enable != 0;
  p->timed_step = false;
  return MUON_OK;
}

muon_status muon_plan_phase_ms(muon_plan *p, float out[3], int32_t *ns_launches) {
  if (!p || !out) { set_error("muon_plan_phase_ms: NULL argument"); return MUON_ERR_INVALID_ARG; }
  if (!p->timed_step) { set_error("muon_plan_phase_ms: no timed step yet"); return MUON_ERR_INVALID_ARG; }
  out[0] = out[1] = out[2] = 0.f;
  for (size_t w = 0; w < p->waves.size(); ++w) {
    hipEvent_t *ev = reinterpret_cast<hipEvent_t *>(&p->phase_events[4 * w]);
    hipError_t e = hipEventSynchronize(ev[3]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (timing)");
    for (int k = 0; k < 3; ++k) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[k], ev[k + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      out[k] += ms;
    }
  }
  if (ns_launches) *ns_launches = p->timed_launches;
  return MUON_OK;
}

void muon_plan_destroy(muon_plan *p) {
  if (!p) return;
  if (p->side_stream) {
    (void)hipStreamSynchronize((hipStream_t)p->side_stream);
    (void)hipStreamDestroy((hipStream_t)p->side_stream);
    (void)hipEventDestroy((hipEvent_t)p->fork_ev);
    (void)hipEventDestroy((hipEvent_t)p->join_ev);
  }
  for (void *ev : p->phase_events) (void)hipEventDestroy((hipEvent_t)ev);
  for (int s = 0; s < 2; ++s) {
    if (p->event_live[s]) (void)hipEventSynchronize((hipEvent_t)p->events[s]);
    if (p->staging[s]) (void)hipHostFree(p->staging[s]);
    if (p->events[s]) (void)hipEventDestroy((hipEvent_t)p->events[s]);
  }
  delete p;
}

}  // extern "C"
