// Internal declarations shared by the libsa HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/sa.h"

namespace sa {

typedef uint16_t bf16_t;

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// round-to-nearest-even float -> bf16 (finite inputs)
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// order-preserving map of a float to uint32 (+0 and -0 map to the same key)
__device__ __forceinline__ uint32_t sortable(float f) {
  f = f + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// wave64 reductions
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// bump allocator over a caller workspace
struct Arena {
  char* base;
  size_t size;
  size_t used;
  __host__ void* take(size_t bytes) {
    size_t off = (used + 255) & ~size_t(255);
    used = off + ((bytes + 255) & ~size_t(255));
    return base ? (void*)(base + off) : nullptr;
  }
  template <typename T> __host__ T* get(size_t count) { return (T*)take(count * sizeof(T)); }
};

// ---------------------------------------------------------------------------
// launchers (host functions, one translation unit each)
// ---------------------------------------------------------------------------

// k_permute.hip --------------------------------------------------------------
// Stable counting sort of labels[h][n] in [0, C): perm (original indices in
// (label, index) order) and offsets [H][C+1].
size_t label_sort_scratch(int H, int N, int C);
hipError_t label_sort(const int32_t* labels, int32_t* perm, int32_t* offsets, int H, int N, int C,
                      Arena& scratch, hipStream_t st);

// x_perm[h][p][:] = x[h][perm[h][p]][:]
hipError_t gather_rows(const void* x, void* x_perm, const int32_t* perm, int H, int N, int d,
                       int dtype, hipStream_t st);

// Member means of columns [col0, col0+dc) of x rows per cluster, fp32, written
// to out[h][c][0..dc) with row stride out_stride.  Empty clusters: keep the
// existing value if keep_empty, else zeros.
// gather_rows and the member means (whole rows, empty clusters -> zero) in
// one pass over the rows, one workgroup per cluster
hipError_t gather_means(const void* x, int dtype, int d, const int32_t* perm, const int32_t* offsets,
                        int H, int N, int C, void* x_perm, float* means, hipStream_t st);
// Rows are summed in runs (one workgroup each) whose partial sums go to
// `scratch` (means_scratch bytes) and are added in run order.
size_t means_scratch(int H, int N, int C, int dc);
hipError_t cluster_means(const void* x, int dtype, int d, int col0, int dc, const int32_t* perm,
                         const int32_t* offsets, int H, int N, int C, float* out, int out_stride,
                         bool keep_empty, float* scratch, hipStream_t st);

// raster block label of every token of a frames x height x width grid for
// blocks of ext[0] x ext[1] x ext[2] tokens (the same labels for every head)
hipError_t raster_labels(int32_t* labels, int H, int frames, int height, int width, const int* ext,
                         hipStream_t st);

// labels[h][perm[h][p]] = cluster of position p, from offsets
hipError_t labels_from_offsets(const int32_t* perm, const int32_t* offsets, int32_t* labels, int H,
                               int N, int C, hipStream_t st);

// k_kmeans.hip ---------------------------------------------------------------
// c[h][j][0..dc) = x[h][j][col0..col0+dc) for j < C (first-k seeding)
hipError_t kmeans_seed(const void* x, int dtype, int d, int col0, int dc, int H, int N, int C,
                       float* c, hipStream_t st);
// labels[h][n] = argmin_j sum_t (x[h][n][col0+t] - c[h][j][t])^2, ties -> smallest j
hipError_t kmeans_assign(const void* x, int dtype, int d, int col0, int dc, int H, int N, int C,
                         const float* c, int32_t* labels, hipStream_t st);
bool kmeans_width_supported(int dc);
// One Lloyd step in one pass over bf16 rows (assignment as kmeans_assign on
// the matrix cores, then per-workgroup cluster sums and counts, added in
// workgroup order): labels of every token, then c[h][j] <- mean of its
// members (unchanged when empty).  `scratch`: kmeans_step_scratch bytes, kept
// between the steps of one run: it carries the centroids' matrix-core terms
// from each step to the next; `first` builds them from c (the first step of a
// run, or after c changed outside the steps).
// With `sort` (whole rows only: col0 = 0, dc = d), the step also writes the
// stable counting sort of its labels (perm, offsets) and x in that order
// (x_perm), as label_sort and gather_rows would, in one extra pass.
struct StepSort {
  int32_t* perm;
  int32_t* offsets;
  void* x_perm;
};
bool kmeans_step_supported(int dtype, const void* x, int d, int col0, int dc, int C);
size_t kmeans_step_scratch(int H, int N, int C, int dc);
// `seed` (with `first`): first-k seeding of c from x inside the step's set-up.
hipError_t kmeans_step(const void* x, int d, int col0, int dc, int H, int N, int C, float* c,
                       int32_t* labels, float* scratch, bool first, bool seed, const StepSort* sort,
                       hipStream_t st);
// labels = (a_t*Cs + a_h)*Cs + a_w
hipError_t combo_labels(const int32_t* sub_labels, int32_t* labels, int H, int N, int Cs,
                        hipStream_t st);
// centroids [H][3*Cs][d]: row s*Cs+c = slice s centroid in its columns, zeros elsewhere
hipError_t expand_sub_centroids(const float* sub, int H, int Cs, int d, const int* dims,
                                float* out, hipStream_t st);
// inverse: compact blocks [3][H][Cs][d_s] from the expanded layout
hipError_t compact_sub_centroids(const float* expanded, int H, int Cs, int d, const int* dims, float* sub,
                                 hipStream_t st);

// k_bisect.hip ---------------------------------------------------------------
size_t bisect_scratch(int H, int N, int d, int leaf);
// Heads below h0 are rows of x0 (order and leaf offsets to perm0 / off0), the
// others of x1 (perm1 / off1); H counts both.  One tensor: x1 = x0, h0 = H.
// With cen0 non-null, the leaf means (fp32 [heads][C][d]) go to cen0 / cen1
// and the rows in cluster order to xp0 / xp1 where those are non-null.
hipError_t bisect_run(const void* x0, const void* x1, int h0, int dtype, int H, int N, int d, int leaf,
                      int iters, int32_t* perm0, int32_t* perm1, int32_t* off0, int32_t* off1, void* xp0,
                      void* xp1, float* cen0, float* cen1, Arena& s, hipStream_t st);

// k_select.hip ---------------------------------------------------------------
struct SelectArgs {
  int H, N, d, Cq, Ck;
  const int32_t* q_off;   // [H][Cq+1]
  const float* qbar;      // [H][Cq][d]
  const int32_t* k_off;   // [H][Ck+1]
  const float* kbar;      // [H][Ck][d] or [H][3*Cs][d] (subspace)
  int subspace, Cs;
  int dims[3];
  double scale;
  double top_p;
  int floor_units, online, weighted;
  uint32_t* mask;         // [H][Cq][W]
  int32_t* counts;        // [H][Cq]
  int32_t* init_counts;   // [H][Cq] or null
  int32_t* head_topk;     // [H]
  // competition domain (cluster mode): SA_DOMAIN_ROW / _HEAD / _GROUP
  int domain, group;
  double max_entropy;
  double* head_entropy;   // [H] or null
  int rule;               // SA_RULE_TOP_P / SA_RULE_STAT
  double stat_lambda;
};
size_t select_scratch(int H, int Cq, int Ck, int subspace, int domain, int group);
hipError_t select_run(const SelectArgs& a, Arena& scratch, hipStream_t st);

// k_attn.hip -----------------------------------------------------------------
struct AttnArgs {
  int H, N, d, Cq, Ck, dtype, tile_rows, compensate;
  int max_tiles;          // upper bound on query tiles per head (0 = derive)
  float scale;
  const void* q_perm;     // [H][N][d] queries in query-cluster order
  const void* q_src;      // if set: [H][N][d] queries in original order, read through q_idx instead
  const int32_t* q_idx;   // [H][N] original index of query position
  const int32_t* q_off;   // [H][Cq+1]
  const void* k_perm;     // [H][N][d]
  const int32_t* k_off;   // [H][Ck+1]
  const float* kbar;      // [H][Ck][d] (compensation)
  const void* v_perm;     // [H][N][d]
  const float* vbar;      // [H][Ck][d] (compensation)
  const uint32_t* mask;   // [H][Cq][W]
  void* o;                // [H][N][d] original order
  hipEvent_t ev_start;    // recorded right before / after the attention
  hipEvent_t ev_stop;     // kernels when not null (caller's timing events)
  float* lse;             // [H][N] original order, natural-log normaliser (optional)
};
size_t attn_scratch(int H, int N, int d, int Cq, int Ck, int tile_rows, int compensate, int dtype,
                    int max_tiles);

// k_attn_bwd.hip --------------------------------------------------------------
struct AttnBwdArgs {
  int H, N, d, Cq, Ck;
  float scale;
  const void* q_perm;     // bf16 [H][N][d] query-cluster order
  const int32_t* q_idx;   // [H][N]
  const int32_t* q_off;   // [H][Cq+1]
  const void* k_perm;     // bf16 [H][N][d] key-cluster order
  const int32_t* k_idx;   // [H][N]
  const int32_t* k_off;   // [H][Ck+1]
  const void* v_perm;     // bf16 [H][N][d] key-cluster order
  const uint32_t* mask;   // [H][Cq][W]
  const void* O;          // bf16 [H][N][d] forward output, original order
  const void* dO;         // bf16 [H][N][d] original order
  const float* lse;       // f32 [H][N] original order, the forward's normaliser (optional)
  float* dq;              // f32 [H][N][d] original order
  float* dk;
  float* dv;
};
size_t attn_bwd_scratch(int H, int N, int d, int Cq, int Ck);
hipError_t attn_bwd_run(const AttnBwdArgs& a, Arena& scratch, hipStream_t st);
hipError_t attn_run(const AttnArgs& a, Arena& scratch, hipStream_t st);

}  // namespace sa
