// C ABI of libsa: argument validation, workspace planning and the launch
// sequence of each entry point.  Nothing here computes on the host beyond
// sizes; every step of the method runs in the kernels of k_*.hip.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sa_internal.h"

using namespace sa;

namespace {

constexpr int KMEANS_MAX = 1024;
constexpr int SUB_MAX = 32;
constexpr int SELECT_MAX = 1024;
constexpr int TILE_MAX = 128;

int esize(int dtype) { return dtype == SA_F32 ? 4 : 2; }

sa_status check_problem(const sa_problem* p) {
  if (!p) return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return SA_ERR_DTYPE;
  if (p->heads < 1 || p->n < 1 || p->frames < 1 || p->height < 1 || p->width < 1)
    return SA_ERR_SHAPE;
  if (int64_t(p->frames) * p->height * p->width != p->n) return SA_ERR_SHAPE;
  if (p->d != 64 && p->d != 128) return SA_ERR_SHAPE;
  if (p->n > (1 << 24) || int64_t(p->heads) * p->n > (int64_t(1) << 31)) return SA_ERR_SHAPE;
  // the kernels address one head's rows of a tensor with 32-bit byte offsets
  if (int64_t(p->n) * p->d * esize(p->dtype) >= (int64_t(1) << 32)) return SA_ERR_SHAPE;
  return SA_OK;
}

int clusters_of(const sa_problem* p, const sa_cluster_cfg* c) {
  switch (c->method) {
    case SA_KMEANS: return c->clusters;
    case SA_BISECT: return c->leaf >= 1 ? ceil_div(p->n, c->leaf) : -1;
    case SA_SUBSPACE: return c->clusters * c->clusters * c->clusters;
    case SA_RASTER:
      for (int k = 0; k < 3; ++k)
        if (c->sub_dims[k] < 1) return -1;
      return ceil_div(p->frames, c->sub_dims[0]) * ceil_div(p->height, c->sub_dims[1]) *
             ceil_div(p->width, c->sub_dims[2]);
    default: return -1;
  }
}

int centroid_rows(const sa_problem* p, const sa_cluster_cfg* c) {
  return c->method == SA_SUBSPACE ? 3 * c->clusters : clusters_of(p, c);
}

sa_status check_cluster_cfg(const sa_problem* p, const sa_cluster_cfg* c) {
  if (!c) return SA_ERR_INVALID_ARG;
  if (c->iters < 1 || c->iters > 1000) return SA_ERR_INVALID_ARG;
  if (c->tile_cap < 0) return SA_ERR_INVALID_ARG;
  if (c->init != SA_INIT_FIRST && c->init != SA_INIT_GIVEN) return SA_ERR_INVALID_ARG;
  switch (c->method) {
    case SA_KMEANS:
      if (c->clusters < 1 || c->clusters > KMEANS_MAX) return SA_ERR_INVALID_ARG;
      if (c->clusters > p->n) return SA_ERR_SHAPE;
      return SA_OK;
    case SA_BISECT:
      if (c->leaf < 4) return SA_ERR_INVALID_ARG;
      if (c->init != SA_INIT_FIRST) return SA_ERR_INVALID_ARG;
      if (ceil_div(p->n, c->leaf) > 65536) return SA_ERR_SHAPE;
      return SA_OK;
    case SA_SUBSPACE: {
      if (c->clusters < 1 || c->clusters > SUB_MAX) return SA_ERR_INVALID_ARG;
      if (c->clusters > p->n) return SA_ERR_SHAPE;
      int sum = 0;
      for (int s = 0; s < 3; ++s) {
        if (!kmeans_width_supported(c->sub_dims[s])) return SA_ERR_UNSUPPORTED;
        sum += c->sub_dims[s];
      }
      if (sum != p->d) return SA_ERR_SHAPE;
      return SA_OK;
    }
    case SA_RASTER: {
      if (c->init != SA_INIT_FIRST) return SA_ERR_INVALID_ARG;
      const int ext[3] = {p->frames, p->height, p->width};
      for (int k = 0; k < 3; ++k)
        if (c->sub_dims[k] < 1 || c->sub_dims[k] > ext[k]) return SA_ERR_INVALID_ARG;
      if (clusters_of(p, c) > 65536) return SA_ERR_SHAPE;
      return SA_OK;
    }
    default: return SA_ERR_INVALID_ARG;
  }
}

sa_status check_attn_cfg(const sa_attn_cfg* c) {
  if (!c) return SA_ERR_INVALID_ARG;
  if (!(c->scale >= 0.f) || !isfinite(c->scale)) return SA_ERR_INVALID_ARG;
  if ((c->ev_start == nullptr) != (c->ev_stop == nullptr)) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

sa_status check_select_cfg(const sa_select_cfg* c) {
  if (!c) return SA_ERR_INVALID_ARG;
  if (!isfinite(c->top_p)) return SA_ERR_INVALID_ARG;
  if (c->rule != SA_RULE_TOP_P && c->rule != SA_RULE_STAT) return SA_ERR_INVALID_ARG;
  if (c->rule == SA_RULE_TOP_P && c->top_p <= 0.0 && c->topk_floor <= 0) return SA_ERR_INVALID_ARG;
  if (c->rule == SA_RULE_STAT && (c->topk_floor < 1 || !isfinite(c->stat_lambda))) return SA_ERR_INVALID_ARG;
  if (c->rule == SA_RULE_STAT && c->domain != SA_DOMAIN_ROW) return SA_ERR_UNSUPPORTED;
  if (c->domain != SA_DOMAIN_ROW && c->domain != SA_DOMAIN_HEAD && c->domain != SA_DOMAIN_GROUP)
    return SA_ERR_INVALID_ARG;
  if (c->domain == SA_DOMAIN_GROUP && (c->group < 1 || !isfinite(c->max_entropy))) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

int tile_rows(const sa_cluster_cfg* q) {
  const int cap = q->tile_cap > 0 ? q->tile_cap : TILE_MAX;
  return std::min(cap, TILE_MAX);
}

int max_tiles(const sa_problem* p, const sa_cluster_cfg* q) {
  const int rows = tile_rows(q);
  const int C = clusters_of(p, q);
  if (q->method == SA_BISECT) return C * ceil_div(q->leaf, rows);
  return p->n / rows + C + 1;
}

// scratch (transient) bytes of each component
size_t cluster_scratch(const sa_problem* p, const sa_cluster_cfg* c) {
  const int H = p->heads, N = p->n;
  switch (c->method) {
    case SA_KMEANS:
      return std::max(means_scratch(H, N, c->clusters, p->d), kmeans_step_scratch(H, N, c->clusters, p->d)) +
             label_sort_scratch(H, N, c->clusters) + 512;
    case SA_BISECT: return bisect_scratch(H, N, p->d, c->leaf) + 256;
    case SA_RASTER: return label_sort_scratch(H, N, clusters_of(p, c)) + 256;
    case SA_SUBSPACE: {
      Arena a{nullptr, 0, 0};
      a.get<int32_t>(size_t(3) * H * N);  // slice labels
      size_t comp = 0;
      for (int s = 0; s < 3; ++s) comp += size_t(H) * c->clusters * c->sub_dims[s];
      a.get<float>(comp);                  // compact slice centroids
      a.get<int32_t>(size_t(H) * N);       // slice perm
      a.get<int32_t>(size_t(H) * (c->clusters + 1));
      size_t ms = 0;
      for (int s = 0; s < 3; ++s)
        ms = std::max(ms, std::max(means_scratch(H, N, c->clusters, c->sub_dims[s]),
                                   kmeans_step_scratch(H, N, c->clusters, c->sub_dims[s])));
      a.take(ms);                          // member-mean run sums or step partials
      return a.used + std::max(label_sort_scratch(H, N, c->clusters),
                               label_sort_scratch(H, N, clusters_of(p, c))) + 256;
    }
  }
  return 0;
}

struct Plan {
  size_t total;
};

// Q and K bisected with the same leaf size and round count form one problem
// of 2H heads: every launch of the bisection covers both tensors.
bool paired_bisect(const sa_cluster_cfg* qc, const sa_cluster_cfg* kc) {
  return qc->method == SA_BISECT && kc->method == SA_BISECT && qc->leaf == kc->leaf &&
         qc->iters == kc->iters;
}

// scratch the two-tensor clustering needs (the paired bisection's, or the
// larger of the two separate ones)
// Q and K clustered separately run side by side, each in its own part
size_t cluster_qk_scratch(const sa_problem* p, const sa_cluster_cfg* qc, const sa_cluster_cfg* kc) {
  return paired_bisect(qc, kc) ? bisect_scratch(2 * p->heads, p->n, p->d, qc->leaf) + 256
                               : cluster_scratch(p, qc) + 256 + cluster_scratch(p, kc);
}

// carve the persistent buffers of sa_forward; null base = size only
struct FwdBufs {
  sa_clusters q, k;
  void* v_perm;
  float* v_means;
  int32_t* counts;
  int32_t* head_topk;
  char* scratch;
  size_t scratch_bytes;
};

FwdBufs carve_forward(const sa_problem* p, const sa_cluster_cfg* qc, const sa_cluster_cfg* kc,
                      const sa_select_cfg* sc, const sa_attn_cfg* ac, char* base, size_t* used) {
  const int H = p->heads, N = p->n, d = p->d;
  const int Cq = clusters_of(p, qc), Ck = clusters_of(p, kc);
  Arena a{base, 0, 0};
  FwdBufs b{};
  auto fill = [&](sa_clusters& c, const sa_cluster_cfg* cfg, int C) {
    c.labels = a.get<int32_t>(size_t(H) * N);
    c.perm = a.get<int32_t>(size_t(H) * N);
    c.offsets = a.get<int32_t>(size_t(H) * (C + 1));
    c.centroids = a.get<float>(size_t(H) * centroid_rows(p, cfg) * d);
    c.x_perm = a.take(size_t(H) * N * d * esize(p->dtype));
  };
  fill(b.q, qc, Cq);
  fill(b.k, kc, Ck);
  b.v_perm = a.take(size_t(H) * N * d * esize(p->dtype));
  b.v_means = (ac && ac->compensate) ? a.get<float>(size_t(H) * Ck * d) : nullptr;
  b.counts = a.get<int32_t>(size_t(H) * Cq);
  b.head_topk = a.get<int32_t>(size_t(H));
  const size_t fixed = a.used;
  size_t scr = cluster_qk_scratch(p, qc, kc);
  scr = std::max(scr, select_scratch(H, Cq, Ck, kc->method == SA_SUBSPACE, sc ? sc->domain : SA_DOMAIN_ROW,
                                     sc ? sc->group : 1) + 256);
  scr = std::max(scr, attn_scratch(H, N, d, Cq, Ck, tile_rows(qc), ac ? ac->compensate : 0,
                                   p->dtype, max_tiles(p, qc)) + 256);
  b.scratch = base ? base + fixed : nullptr;
  b.scratch_bytes = scr;
  *used = fixed + scr;
  return b;
}

sa_status hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

// ---------------------------------------------------------------------------
// component implementations (arguments already validated)
// ---------------------------------------------------------------------------
// after the bisection proper: labels (the subtree phase has already written
// the member means and the rows in cluster order)
sa_status bisect_tail(const sa_problem* p, const sa_cluster_cfg* c, sa_clusters* out, hipStream_t st) {
  const int H = p->heads, N = p->n;
  const int C = clusters_of(p, c);
  out->num_clusters = C;
  out->method = c->method;
  out->sub_clusters = 0;
  for (int k = 0; k < 3; ++k) out->sub_dims[k] = 0;
  return hip_status(labels_from_offsets(out->perm, out->offsets, out->labels, H, N, C, st));
}

// q_rows false: Q's rows in cluster order are not written (sa_forward's
// attention reads Q through the permutation); its means are.
sa_status do_cluster_pair(const sa_problem* p, const sa_cluster_cfg* qc, const sa_cluster_cfg* kc,
                          const void* q, const void* k, sa_clusters* qo, sa_clusters* ko, Arena& s,
                          hipStream_t st, bool q_rows = true) {
  const int H = p->heads;
  Arena tmp = s;
  const hipError_t e = bisect_run(q, k, H, p->dtype, 2 * H, p->n, p->d, qc->leaf, qc->iters, qo->perm,
                                  ko->perm, qo->offsets, ko->offsets, q_rows ? qo->x_perm : nullptr, ko->x_perm,
                                  qo->centroids, ko->centroids, tmp, st);
  if (e != hipSuccess) return SA_ERR_HIP;
  sa_status r = bisect_tail(p, qc, qo, st);
  if (r == SA_OK) r = bisect_tail(p, kc, ko, st);
  return r;
}

// rows false: a bisection writes the means but not the rows in cluster order
sa_status do_cluster(const sa_problem* p, const sa_cluster_cfg* c, const void* x, sa_clusters* out,
                     Arena& s, hipStream_t st, bool rows = true) {
  const int H = p->heads, N = p->n, d = p->d, dt = p->dtype;
  const int C = clusters_of(p, c);
  hipError_t e = hipSuccess;
  out->num_clusters = C;
  out->method = c->method;
  out->sub_clusters = c->method == SA_SUBSPACE ? c->clusters : 0;
  for (int k = 0; k < 3; ++k) out->sub_dims[k] = c->method == SA_SUBSPACE ? c->sub_dims[k] : 0;
  if (c->method == SA_KMEANS) {
    const bool fused = kmeans_step_supported(dt, x, d, 0, d, C);
    // the fused step seeds inside its first set-up
    const bool seed = c->init == SA_INIT_FIRST;
    if (seed && !fused) e = kmeans_seed(x, dt, d, 0, d, H, N, C, out->centroids, st);
    for (int it = 0; it < c->iters && e == hipSuccess; ++it) {
      Arena tmp = s;
      if (fused) {
        // the last step also sorts the labels and permutes the rows
        float* ksc = (float*)tmp.take(kmeans_step_scratch(H, N, C, d));
        const StepSort so{out->perm, out->offsets, out->x_perm};
        e = kmeans_step(x, d, 0, d, H, N, C, out->centroids, out->labels, ksc, it == 0, it == 0 && seed,
                        it + 1 == c->iters ? &so : nullptr, st);
        if (e == hipSuccess && it + 1 == c->iters) return hip_status(e);
        continue;
      }
      float* msc = (float*)tmp.take(means_scratch(H, N, C, d));
      e = kmeans_assign(x, dt, d, 0, d, H, N, C, out->centroids, out->labels, st);
      if (e == hipSuccess) e = label_sort(out->labels, out->perm, out->offsets, H, N, C, tmp, st);
      if (e == hipSuccess)
        e = cluster_means(x, dt, d, 0, d, out->perm, out->offsets, H, N, C, out->centroids, d, true, msc, st);
    }
  } else if (c->method == SA_RASTER) {
    // block labels from the grid, then the same counting sort and one pass of
    // row gather + member means as the bisection's outputs
    e = raster_labels(out->labels, H, p->frames, p->height, p->width, c->sub_dims, st);
    Arena tmp = s;
    if (e == hipSuccess) e = label_sort(out->labels, out->perm, out->offsets, H, N, C, tmp, st);
    if (e == hipSuccess) e = gather_means(x, dt, d, out->perm, out->offsets, H, N, C, out->x_perm, out->centroids, st);
    return hip_status(e);
  } else if (c->method == SA_BISECT) {
    Arena tmp = s;
    void* xp = rows ? out->x_perm : nullptr;
    e = bisect_run(x, x, H, dt, H, N, d, c->leaf, c->iters, out->perm, out->perm, out->offsets,
                   out->offsets, xp, xp, out->centroids, out->centroids, tmp, st);
    if (e == hipSuccess) return bisect_tail(p, c, out, st);
  } else {
    const int Cs = c->clusters;
    Arena tmp = s;
    int32_t* sub_labels = tmp.get<int32_t>(size_t(3) * H * N);
    size_t comp = 0;
    for (int k = 0; k < 3; ++k) comp += size_t(H) * Cs * c->sub_dims[k];
    float* sub_c = tmp.get<float>(comp);
    int32_t* sperm = tmp.get<int32_t>(size_t(H) * N);
    int32_t* soff = tmp.get<int32_t>(size_t(H) * (Cs + 1));
    size_t ms = 0;
    for (int k = 0; k < 3; ++k)
      ms = std::max(ms, std::max(means_scratch(H, N, Cs, c->sub_dims[k]),
                                 kmeans_step_scratch(H, N, Cs, c->sub_dims[k])));
    float* msc = (float*)tmp.take(ms);
    // SA_INIT_GIVEN: every slice starts from the centroids already in
    // out->centroids (expanded layout)
    if (c->init == SA_INIT_GIVEN) e = compact_sub_centroids(out->centroids, H, Cs, d, c->sub_dims, sub_c, st);
    size_t coff = 0;
    int col0 = 0;
    for (int k = 0; k < 3 && e == hipSuccess; ++k) {
      const int ds = c->sub_dims[k];
      float* cs = sub_c + coff;
      int32_t* lab = sub_labels + size_t(k) * H * N;
      const bool fused = kmeans_step_supported(dt, x, d, col0, ds, Cs);
      const bool seed = c->init == SA_INIT_FIRST;
      if (seed && !fused) e = kmeans_seed(x, dt, d, col0, ds, H, N, Cs, cs, st);
      for (int it = 0; it < c->iters && e == hipSuccess; ++it) {
        Arena t2 = tmp;
        if (fused) {
          e = kmeans_step(x, d, col0, ds, H, N, Cs, cs, lab, msc, it == 0, it == 0 && seed, nullptr, st);
          continue;
        }
        e = kmeans_assign(x, dt, d, col0, ds, H, N, Cs, cs, lab, st);
        if (e == hipSuccess) e = label_sort(lab, sperm, soff, H, N, Cs, t2, st);
        if (e == hipSuccess)
          e = cluster_means(x, dt, d, col0, ds, sperm, soff, H, N, Cs, cs, ds, true, msc, st);
      }
      coff += size_t(H) * Cs * ds;
      col0 += ds;
    }
    if (e == hipSuccess) e = combo_labels(sub_labels, out->labels, H, N, Cs, st);
    if (e == hipSuccess) {
      Arena t2 = tmp;
      e = label_sort(out->labels, out->perm, out->offsets, H, N, C, t2, st);
    }
    if (e == hipSuccess) e = expand_sub_centroids(sub_c, H, Cs, d, c->sub_dims, out->centroids, st);
  }
  if (e == hipSuccess) e = gather_rows(x, out->x_perm, out->perm, H, N, d, dt, st);
  return hip_status(e);
}

// Q and K clustered separately (different methods or settings) are two chains
// of mostly short launches: K's runs on a second stream of the device (default
// priority, created on first use), forked from the caller's stream and joined
// back to it with events, so the two chains overlap.  The record/wait pairs
// of one call are made under a lock, so calls on distinct workspaces stay
// independent.
constexpr int MAX_DEVICES = 64;
struct ForkJoin {
  hipStream_t s2;
  hipEvent_t fork, join;
};
std::mutex g_fork_mu;
ForkJoin g_fork[MAX_DEVICES];

// enqueue a(st) and b(s2) side by side: s2 starts after the work already on
// st, and st continues after both
template <typename A, typename B>
sa_status side_by_side(hipStream_t st, A&& a, B&& b) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_fork_mu);
  ForkJoin& f = g_fork[dev];
  if (!f.s2) {
    ForkJoin n{};
    if (hipStreamCreateWithFlags(&n.s2, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess) {
      // release what was made, so that a later call starts over
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s2) (void)hipStreamDestroy(n.s2);
      return SA_ERR_HIP;
    }
    f = n;
  }
  if (hipEventRecord(f.fork, st) != hipSuccess || hipStreamWaitEvent(f.s2, f.fork, 0) != hipSuccess)
    return SA_ERR_HIP;
  sa_status r = a(st);
  const sa_status rb = b(f.s2);
  // joined whatever happened, so that later work on the caller's stream
  // follows everything enqueued on the second one
  const bool joined = hipEventRecord(f.join, f.s2) == hipSuccess && hipStreamWaitEvent(st, f.join, 0) == hipSuccess;
  if (r == SA_OK) r = rb;
  if (r == SA_OK && !joined) r = SA_ERR_HIP;
  return r;
}

sa_status do_cluster_qk(const sa_problem* p, const sa_cluster_cfg* qc, const sa_cluster_cfg* kc,
                        const void* q, const void* k, sa_clusters* qo, sa_clusters* ko, Arena& s,
                        hipStream_t st, bool q_rows = true) {
  if (paired_bisect(qc, kc)) return do_cluster_pair(p, qc, kc, q, k, qo, ko, s, st, q_rows);
  Arena sk = s;  // K's scratch follows Q's
  sk.take(cluster_scratch(p, qc));
  return side_by_side(
      st, [&](hipStream_t x) { return do_cluster(p, qc, q, qo, s, x, q_rows); },
      [&](hipStream_t x) { return do_cluster(p, kc, k, ko, sk, x); });
}

sa_status do_select(const sa_problem* p, const sa_select_cfg* c, const sa_clusters* q,
                    const sa_clusters* k, uint32_t* mask, int32_t* counts, int32_t* init_counts,
                    int32_t* head_topk, double* head_entropy, Arena& s, hipStream_t st) {
  SelectArgs a{};
  a.H = p->heads;
  a.N = p->n;
  a.d = p->d;
  a.Cq = q->num_clusters;
  a.Ck = k->num_clusters;
  a.q_off = q->offsets;
  a.qbar = q->centroids;
  a.k_off = k->offsets;
  a.kbar = k->centroids;
  a.subspace = k->method == SA_SUBSPACE;
  a.Cs = k->sub_clusters;
  for (int i = 0; i < 3; ++i) a.dims[i] = k->sub_dims[i];
  a.scale = 1.0 / sqrt(double(p->d));
  a.top_p = c->top_p;
  a.floor_units = c->topk_floor;
  a.online = c->online_topk != 0;
  a.weighted = c->size_weighted != 0;
  a.mask = mask;
  a.counts = counts;
  a.init_counts = init_counts;
  a.head_topk = head_topk;
  a.domain = c->domain;
  a.group = c->group;
  a.max_entropy = c->max_entropy;
  a.head_entropy = head_entropy;
  a.rule = c->rule;
  a.stat_lambda = c->stat_lambda;
  Arena tmp = s;
  return hip_status(select_run(a, tmp, st));
}

sa_status do_attn(const sa_problem* p, const sa_attn_cfg* c, const sa_clusters* q,
                  const sa_clusters* k, const void* v_perm, const float* v_means,
                  const uint32_t* mask, void* o, int rows, int maxt, Arena& s, hipStream_t st,
                  const void* q_src = nullptr) {
  AttnArgs a{};
  a.H = p->heads;
  a.N = p->n;
  a.d = p->d;
  a.Cq = q->num_clusters;
  a.Ck = k->num_clusters;
  a.dtype = p->dtype;
  a.tile_rows = rows;
  a.max_tiles = maxt;
  a.compensate = c->compensate != 0;
  a.scale = c->scale > 0.f ? c->scale : float(1.0 / sqrt(double(p->d)));
  a.q_perm = q->x_perm;
  a.q_src = q_src;  // set: query rows from the original order through q_idx
  a.q_idx = q->perm;
  a.q_off = q->offsets;
  a.k_perm = k->x_perm;
  a.k_off = k->offsets;
  a.kbar = k->centroids;
  a.v_perm = v_perm;
  a.vbar = v_means;
  a.mask = mask;
  a.o = o;
  a.ev_start = static_cast<hipEvent_t>(c->ev_start);
  a.ev_stop = static_cast<hipEvent_t>(c->ev_stop);
  a.lse = static_cast<float*>(c->lse);
  Arena tmp = s;
  return hip_status(attn_run(a, tmp, st));
}

// ---------------------------------------------------------------------------
// Library-owned attention scratch for sa_block_sparse_attn_noalloc: one array
// per GPU in the code object, so that entry point allocates nothing.  In host
// code `scratch` only names the symbol; its device address on the current GPU
// comes from hipGetSymbolAddress (once per device) and only that address is
// handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(SA_NOALLOC_ATTN_SCRATCH_BYTES);
__device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// device address of the current GPU's scratch array (looked up on first use)
sa_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

bool clusters_ok(const sa_clusters* c, bool need_xperm) {
  return c && c->perm && c->offsets && c->centroids && (!need_xperm || c->x_perm) &&
         c->num_clusters >= 1;
}

}  // namespace

extern "C" {

SA_API int32_t sa_num_clusters(const sa_problem* p, const sa_cluster_cfg* cfg) {
  if (check_problem(p) != SA_OK || check_cluster_cfg(p, cfg) != SA_OK) return -1;
  return clusters_of(p, cfg);
}

SA_API sa_status sa_workspace_size(const sa_problem* p, const sa_cluster_cfg* qcfg,
                                   const sa_cluster_cfg* kcfg, const sa_select_cfg* scfg,
                                   const sa_attn_cfg* acfg, size_t* bytes) {
  if (!bytes) return SA_ERR_INVALID_ARG;
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (qcfg && (st = check_cluster_cfg(p, qcfg)) != SA_OK) return st;
  if (kcfg && (st = check_cluster_cfg(p, kcfg)) != SA_OK) return st;
  if (qcfg && kcfg) {
    size_t used = 0;
    carve_forward(p, qcfg, kcfg, scfg, acfg, nullptr, &used);
    *bytes = used + 256;
    return SA_OK;
  }
  size_t b = 256;
  if (qcfg) b = std::max(b, cluster_scratch(p, qcfg));
  if (kcfg) b = std::max(b, cluster_scratch(p, kcfg));
  *bytes = b + 256;
  return SA_OK;
}

SA_API sa_status sa_cluster(const sa_problem* p, const sa_cluster_cfg* cfg, const void* x,
                            sa_clusters* out, void* ws, size_t ws_bytes, void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if ((st = check_cluster_cfg(p, cfg)) != SA_OK) return st;
  if (!x || !out || !out->labels || !out->perm || !out->offsets || !out->centroids || !out->x_perm)
    return SA_ERR_INVALID_ARG;
  if (!ws) return SA_ERR_INVALID_ARG;
  if (ws_bytes < cluster_scratch(p, cfg)) return SA_ERR_WORKSPACE;
  Arena s{(char*)ws, ws_bytes, 0};
  return do_cluster(p, cfg, x, out, s, (hipStream_t)stream);
}

SA_API sa_status sa_cluster_qk(const sa_problem* p, const sa_cluster_cfg* qcfg,
                               const sa_cluster_cfg* kcfg, const void* q, const void* k,
                               sa_clusters* qout, sa_clusters* kout, void* ws, size_t ws_bytes,
                               void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if ((st = check_cluster_cfg(p, qcfg)) != SA_OK) return st;
  if ((st = check_cluster_cfg(p, kcfg)) != SA_OK) return st;
  for (const sa_clusters* c : {qout, kout})
    if (!c || !c->labels || !c->perm || !c->offsets || !c->centroids || !c->x_perm) return SA_ERR_INVALID_ARG;
  if (!q || !k || !ws) return SA_ERR_INVALID_ARG;
  if (ws_bytes < cluster_qk_scratch(p, qcfg, kcfg)) return SA_ERR_WORKSPACE;
  Arena s{(char*)ws, ws_bytes, 0};
  return do_cluster_qk(p, qcfg, kcfg, q, k, qout, kout, s, (hipStream_t)stream);
}

SA_API sa_status sa_permute(const sa_problem* p, const sa_clusters* c, const void* x, void* x_perm,
                            float* means, void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (!clusters_ok(c, false) || !x || !x_perm) return SA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = means ? gather_means(x, p->dtype, p->d, c->perm, c->offsets, p->heads, p->n,
                                             c->num_clusters, x_perm, means, s)
                             : gather_rows(x, x_perm, c->perm, p->heads, p->n, p->d, p->dtype, s);
  return hip_status(e);
}

SA_API sa_status sa_select(const sa_problem* p, const sa_select_cfg* cfg, const sa_clusters* q,
                           const sa_clusters* k, uint32_t* mask, int32_t* counts,
                           int32_t* init_counts, int32_t* head_topk, double* head_entropy, void* ws,
                           size_t ws_bytes, void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if ((st = check_select_cfg(cfg)) != SA_OK) return st;
  if (!clusters_ok(q, false) || !clusters_ok(k, false) || !mask || !counts || !head_topk || !ws)
    return SA_ERR_INVALID_ARG;
  const int sub = k->method == SA_SUBSPACE;
  if (sub && (k->sub_clusters < 1 || k->sub_clusters > SUB_MAX ||
              k->sub_dims[0] + k->sub_dims[1] + k->sub_dims[2] != p->d))
    return SA_ERR_INVALID_ARG;
  if (!sub && k->num_clusters > SELECT_MAX) return SA_ERR_UNSUPPORTED;
  if (sub && (cfg->domain != SA_DOMAIN_ROW || cfg->rule != SA_RULE_TOP_P)) return SA_ERR_UNSUPPORTED;
  if (ws_bytes < select_scratch(p->heads, q->num_clusters, k->num_clusters, sub, cfg->domain, cfg->group) + 256)
    return SA_ERR_WORKSPACE;
  Arena s{(char*)ws, ws_bytes, 0};
  return do_select(p, cfg, q, k, mask, counts, init_counts, head_topk, head_entropy, s, (hipStream_t)stream);
}

SA_API sa_status sa_block_sparse_attn(const sa_problem* p, const sa_attn_cfg* cfg,
                                      const sa_clusters* q, const sa_clusters* k,
                                      const void* v_perm, const float* v_means,
                                      const uint32_t* mask, void* o, void* ws, size_t ws_bytes,
                                      void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (!cfg || !clusters_ok(q, true) || !clusters_ok(k, true) || !v_perm || !mask || !o || !ws)
    return SA_ERR_INVALID_ARG;
  if ((st = check_attn_cfg(cfg)) != SA_OK) return st;
  if (cfg->compensate && !v_means) return SA_ERR_INVALID_ARG;
  if (cfg->compensate && k->method == SA_SUBSPACE) return SA_ERR_UNSUPPORTED;
  const int rows = TILE_MAX;
  const int maxt = p->n / rows + q->num_clusters + 1;
  const size_t need = attn_scratch(p->heads, p->n, p->d, q->num_clusters, k->num_clusters, rows,
                                   cfg->compensate, p->dtype, maxt) + 256;
  if (ws_bytes < need) return SA_ERR_WORKSPACE;
  Arena s{(char*)ws, ws_bytes, 0};
  return do_attn(p, cfg, q, k, v_perm, v_means, mask, o, rows, maxt, s, (hipStream_t)stream);
}

SA_API sa_status sa_block_sparse_attn_noalloc(const sa_problem* p, const sa_attn_cfg* cfg,
                                              const sa_clusters* q, const sa_clusters* k,
                                              const void* v_perm, const float* v_means,
                                              const uint32_t* mask, void* o, void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (!cfg || !clusters_ok(q, true) || !clusters_ok(k, true) || !v_perm || !mask || !o)
    return SA_ERR_INVALID_ARG;
  if ((st = check_attn_cfg(cfg)) != SA_OK) return st;
  if (cfg->compensate && !v_means) return SA_ERR_INVALID_ARG;
  if (cfg->compensate && k->method == SA_SUBSPACE) return SA_ERR_UNSUPPORTED;
  const int rows = TILE_MAX;
  const int maxt = p->n / rows + q->num_clusters + 1;
  const size_t need = attn_scratch(p->heads, p->n, p->d, q->num_clusters, k->num_clusters, rows,
                                   cfg->compensate, p->dtype, maxt);
  if (need > NOALLOC_SCRATCH_BYTES) return SA_ERR_WORKSPACE;
  void* base = nullptr;
  if ((st = device_scratch(&base)) != SA_OK) return st;
  Arena s{(char*)base, NOALLOC_SCRATCH_BYTES, 0};
  return do_attn(p, cfg, q, k, v_perm, v_means, mask, o, rows, maxt, s, (hipStream_t)stream);
}

SA_API sa_status sa_block_sparse_attn_bwd_workspace_size(const sa_problem* p, int32_t q_clusters,
                                                         int32_t k_clusters, size_t* bytes) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (!bytes || q_clusters < 1 || k_clusters < 1) return SA_ERR_INVALID_ARG;
  *bytes = attn_bwd_scratch(p->heads, p->n, p->d, q_clusters, k_clusters) + 256;
  return SA_OK;
}

SA_API sa_status sa_block_sparse_attn_bwd(const sa_problem* p, const sa_attn_cfg* cfg,
                                          const sa_clusters* q, const sa_clusters* k,
                                          const void* v_perm, const uint32_t* mask, const void* o,
                                          const void* d_o, const float* lse, float* dq, float* dk,
                                          float* dv, void* ws, size_t ws_bytes, void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if (p->dtype != SA_BF16) return SA_ERR_DTYPE;
  if (!cfg || !clusters_ok(q, true) || !clusters_ok(k, true) || !v_perm || !mask || !o || !d_o || !dq || !dk ||
      !dv || !ws)
    return SA_ERR_INVALID_ARG;
  if ((st = check_attn_cfg(cfg)) != SA_OK) return st;
  if (cfg->compensate) return SA_ERR_UNSUPPORTED;
  if (ws_bytes < attn_bwd_scratch(p->heads, p->n, p->d, q->num_clusters, k->num_clusters) + 256)
    return SA_ERR_WORKSPACE;
  AttnBwdArgs a{};
  a.H = p->heads;
  a.N = p->n;
  a.d = p->d;
  a.Cq = q->num_clusters;
  a.Ck = k->num_clusters;
  a.scale = cfg->scale > 0.f ? cfg->scale : float(1.0 / sqrt(double(p->d)));
  a.q_perm = q->x_perm;
  a.q_idx = q->perm;
  a.q_off = q->offsets;
  a.k_perm = k->x_perm;
  a.k_idx = k->perm;
  a.k_off = k->offsets;
  a.v_perm = v_perm;
  a.mask = mask;
  a.O = o;
  a.dO = d_o;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  Arena s{(char*)ws, ws_bytes, 0};
  return hip_status(attn_bwd_run(a, s, (hipStream_t)stream));
}

SA_API sa_status sa_forward(const sa_problem* p, const sa_cluster_cfg* qcfg,
                            const sa_cluster_cfg* kcfg, const sa_select_cfg* scfg,
                            const sa_attn_cfg* acfg, const void* q, const void* k, const void* v,
                            void* o, uint32_t* mask, void* ws, size_t ws_bytes, void* stream) {
  sa_status st = check_problem(p);
  if (st != SA_OK) return st;
  if ((st = check_cluster_cfg(p, qcfg)) != SA_OK) return st;
  if ((st = check_cluster_cfg(p, kcfg)) != SA_OK) return st;
  if ((st = check_select_cfg(scfg)) != SA_OK) return st;
  if ((st = check_attn_cfg(acfg)) != SA_OK) return st;
  if (!q || !k || !v || !o || !mask || !ws) return SA_ERR_INVALID_ARG;
  if (qcfg->method == SA_SUBSPACE) return SA_ERR_INVALID_ARG;
  if (qcfg->init != SA_INIT_FIRST || kcfg->init != SA_INIT_FIRST) return SA_ERR_INVALID_ARG;
  if (kcfg->method == SA_SUBSPACE && acfg->compensate) return SA_ERR_UNSUPPORTED;
  if (kcfg->method == SA_SUBSPACE && (scfg->domain != SA_DOMAIN_ROW || scfg->rule != SA_RULE_TOP_P))
    return SA_ERR_UNSUPPORTED;
  if (kcfg->method != SA_SUBSPACE && clusters_of(p, kcfg) > SELECT_MAX) return SA_ERR_UNSUPPORTED;
  size_t used = 0;
  carve_forward(p, qcfg, kcfg, scfg, acfg, nullptr, &used);
  if (ws_bytes < used) return SA_ERR_WORKSPACE;
  FwdBufs b = carve_forward(p, qcfg, kcfg, scfg, acfg, (char*)ws, &used);
  hipStream_t s = (hipStream_t)stream;
  Arena scr{b.scratch, b.scratch_bytes, 0};
  // the attention reads Q through the query-cluster permutation, so no
  // cluster-order copy of Q is written (a bisection skips it)
  if ((st = do_cluster_qk(p, qcfg, kcfg, q, k, &b.q, &b.k, scr, s, false)) != SA_OK) return st;
  const hipError_t e = b.v_means ? gather_means(v, p->dtype, p->d, b.k.perm, b.k.offsets, p->heads, p->n,
                                                b.k.num_clusters, b.v_perm, b.v_means, s)
                                 : gather_rows(v, b.v_perm, b.k.perm, p->heads, p->n, p->d, p->dtype, s);
  if (e != hipSuccess) return SA_ERR_HIP;
  if ((st = do_select(p, scfg, &b.q, &b.k, mask, b.counts, nullptr, b.head_topk, nullptr, scr, s)) != SA_OK)
    return st;
  return do_attn(p, acfg, &b.q, &b.k, b.v_perm, b.v_means, mask, o, tile_rows(qcfg),
                 max_tiles(p, qcfg), scr, s, q);
}

SA_API const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case SA_ERR_DTYPE: return "unsupported dtype";
    case SA_ERR_WORKSPACE: return "workspace too small";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

}  // extern "C"
