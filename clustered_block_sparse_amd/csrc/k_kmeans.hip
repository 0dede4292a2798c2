// k-means assignment (and seeding) for query/key clustering and for SCOPE's
// per-subspace key clustering (SCOPE, technical framework: the t/h/w slices
// of the post-RoPE keys are clustered independently).
//
// Distances are evaluated directly as sum_t (x_t - c_t)^2 in fp32 (no
// ||c||^2 - 2 x.c expansion, so no cancellation); ties go to the smallest
// centroid index.  The data here is small next to attention (at most a few
// GFLOP per layer), so the kernel keeps centroid chunks in LDS and token rows
// in registers rather than using matrix cores: the work is two vector ALU
// operations per (token, centroid, dimension).

#include "sa_internal.h"

namespace sa {

namespace {

// One token per lane: the token's slice sits in registers, and every lane of
// the workgroup walks the same centroids in ascending order, so each centroid
// element is one LDS read that the whole wave shares (a broadcast).  Four
// centroids are evaluated at once for instruction-level parallelism; each
// distance is still sum_t (x_t - c_t)^2 accumulated over t in order, and the
// four are compared in index order, so the smallest index wins ties.
template <int DC>
constexpr int cchunk() {
  return DC >= 128 ? 64 : 128;  // centroids per LDS chunk (at most 32 KB)
}

template <typename T, int DC, bool VEC>
__global__ __launch_bounds__(256) void assign_kernel(const T* __restrict__ x, int d, int col0, int N,
                                                     int C, const float* __restrict__ cent,
                                                     int32_t* __restrict__ labels) {
  constexpr int CCH = cchunk<DC>();
  __shared__ __attribute__((aligned(16))) float cs[CCH * DC];
  const int h = blockIdx.y;
  const int tok = blockIdx.x * 256 + threadIdx.x;
  const bool valid = tok < N;
  const T* row = x + (size_t(h) * N + (valid ? tok : 0)) * d + col0;
  float xr[DC];
  if constexpr (VEC) {
    constexpr int EPV = 16 / int(sizeof(T));  // elements per 16-byte vector
#pragma unroll
    for (int q = 0; q < DC / EPV; ++q) {
      const uint4 u = reinterpret_cast<const uint4*>(row)[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) xr[4 * q + e] = __uint_as_float(w[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xr[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
          xr[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < DC; ++t) xr[t] = to_f(row[t]);
  }
  float best = __builtin_huge_valf();
  int bj = 0x7fffffff;
  const float* ch = cent + size_t(h) * C * DC;
  for (int j0 = 0; j0 < C; j0 += CCH) {
    const int nj = min(CCH, C - j0);
    __syncthreads();
    for (int i = threadIdx.x; i < nj * DC; i += 256) cs[i] = ch[size_t(j0) * DC + i];
    __syncthreads();
    int jj = 0;
    for (; jj + 4 <= nj; jj += 4) {
      float dist[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DC; t += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 c4 = *reinterpret_cast<const float4*>(cs + (jj + u) * DC + t);
          float df = xr[t] - c4.x;
          dist[u] = fmaf(df, df, dist[u]);
          df = xr[t + 1] - c4.y;
          dist[u] = fmaf(df, df, dist[u]);
          df = xr[t + 2] - c4.z;
          dist[u] = fmaf(df, df, dist[u]);
          df = xr[t + 3] - c4.w;
          dist[u] = fmaf(df, df, dist[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (dist[u] < best) {
          best = dist[u];
          bj = j0 + jj + u;
        }
    }
    for (; jj < nj; ++jj) {
      float dist = 0.f;
#pragma unroll
      for (int t = 0; t < DC; ++t) {
        const float df = xr[t] - cs[jj * DC + t];
        dist = fmaf(df, df, dist);
      }
      if (dist < best) {
        best = dist;
        bj = j0 + jj;
      }
    }
  }
  if (valid) labels[size_t(h) * N + tok] = bj;
}

template <typename T>
__global__ void seed_kernel(const T* __restrict__ x, int d, int col0, int dc, int N, int C,
                            float* __restrict__ c) {
  const int h = blockIdx.y, j = blockIdx.x;
  for (int t = threadIdx.x; t < dc; t += blockDim.x)
    c[(size_t(h) * C + j) * dc + t] = to_f(x[(size_t(h) * N + j) * d + col0 + t]);
}

__global__ void combo_kernel(const int32_t* __restrict__ sub, int32_t* __restrict__ labels, int H,
                             int N, int Cs) {
  const int h = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const size_t HN = size_t(H) * N;
  const size_t i = size_t(h) * N + n;
  labels[i] = (sub[i] * Cs + sub[HN + i]) * Cs + sub[2 * HN + i];
}

__global__ void expand_kernel(const float* __restrict__ sub, int H, int Cs, int d, int d0, int d1,
                              int d2, float* __restrict__ out) {
  // sub holds three compact blocks: [3][H][Cs][d_s]
  const int h = blockIdx.y, row = blockIdx.x;  // row in [0, 3*Cs)
  const int s = row / Cs, c = row % Cs;
  const int ds[3] = {d0, d1, d2};
  const int off[3] = {0, d0, d0 + d1};
  size_t base = 0;
  for (int q = 0; q < s; ++q) base += size_t(H) * Cs * ds[q];
  const float* src = sub + base + (size_t(h) * Cs + c) * ds[s];
  float* dst = out + (size_t(h) * 3 * Cs + row) * d;
  for (int t = threadIdx.x; t < d; t += blockDim.x) {
    const int u = t - off[s];
    dst[t] = (u >= 0 && u < ds[s]) ? src[u] : 0.f;
  }
}

template <typename T, int DC>
hipError_t assign_launch(const void* x, int d, int col0, int H, int N, int C, const float* c,
                         int32_t* labels, hipStream_t st) {
  dim3 g(ceil_div(N, 256), H);
  // 16-byte row loads need the base, the row pitch and the slice start aligned
  const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (size_t(d) * sizeof(T)) % 16 == 0 &&
                   (size_t(col0) * sizeof(T)) % 16 == 0 && (DC * sizeof(T)) % 16 == 0;
  if (vec)
    assign_kernel<T, DC, true><<<g, 256, 0, st>>>((const T*)x, d, col0, N, C, c, labels);
  else
    assign_kernel<T, DC, false><<<g, 256, 0, st>>>((const T*)x, d, col0, N, C, c, labels);
  return hipGetLastError();
}

template <typename T>
hipError_t assign_dispatch(const void* x, int d, int col0, int dc, int H, int N, int C,
                           const float* c, int32_t* labels, hipStream_t st) {
  switch (dc) {
    case 16: return assign_launch<T, 16>(x, d, col0, H, N, C, c, labels, st);
    case 24: return assign_launch<T, 24>(x, d, col0, H, N, C, c, labels, st);
    case 32: return assign_launch<T, 32>(x, d, col0, H, N, C, c, labels, st);
    case 48: return assign_launch<T, 48>(x, d, col0, H, N, C, c, labels, st);
    case 64: return assign_launch<T, 64>(x, d, col0, H, N, C, c, labels, st);
    case 128: return assign_launch<T, 128>(x, d, col0, H, N, C, c, labels, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool kmeans_width_supported(int dc) {
  return dc == 16 || dc == 24 || dc == 32 || dc == 48 || dc == 64 || dc == 128;
}

hipError_t kmeans_seed(const void* x, int dtype, int d, int col0, int dc, int H, int N, int C,
                       float* c, hipStream_t st) {
  dim3 g(C, H);
  if (dtype == SA_F32)
    seed_kernel<float><<<g, 128, 0, st>>>((const float*)x, d, col0, dc, N, C, c);
  else
    seed_kernel<bf16_t><<<g, 128, 0, st>>>((const bf16_t*)x, d, col0, dc, N, C, c);
  return hipGetLastError();
}

hipError_t kmeans_assign(const void* x, int dtype, int d, int col0, int dc, int H, int N, int C,
                         const float* c, int32_t* labels, hipStream_t st) {
  if (dtype == SA_F32) return assign_dispatch<float>(x, d, col0, dc, H, N, C, c, labels, st);
  return assign_dispatch<bf16_t>(x, d, col0, dc, H, N, C, c, labels, st);
}

hipError_t combo_labels(const int32_t* sub_labels, int32_t* labels, int H, int N, int Cs,
                        hipStream_t st) {
  combo_kernel<<<dim3(ceil_div(N, 256), H), 256, 0, st>>>(sub_labels, labels, H, N, Cs);
  return hipGetLastError();
}

hipError_t expand_sub_centroids(const float* sub, int H, int Cs, int d, const int* dims, float* out,
                                hipStream_t st) {
  expand_kernel<<<dim3(3 * Cs, H), 128, 0, st>>>(sub, H, Cs, d, dims[0], dims[1], dims[2], out);
  return hipGetLastError();
}

}  // namespace sa
