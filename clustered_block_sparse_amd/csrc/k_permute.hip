// Counting-sort permutation into cluster order, row gather and cluster means.
//
// The permutation puts every cluster's tokens in one contiguous range
// (ascending original index inside a cluster), so that a cluster is a dense
// block of rows for block-sparse attention (ClusterAttention, English
// abstract: cluster sizes chosen so block-sparse attention runs at dense
// speed).  The sort is a stable LSD radix sort on 8-bit digits of the label;
// every count is an integer, so the result is exact and deterministic.

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int SORT_CHUNK = 2048;  // elements per workgroup in the sort passes

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << __lane_id()) - 1;
}

// per-chunk digit histogram -> chist[h][digit][chunk]
__global__ __launch_bounds__(256) void sort_hist(const int32_t* __restrict__ keys, int N, int shift,
                                                 int nchunks, int32_t* __restrict__ chist) {
  __shared__ int hist[256];
  const int h = blockIdx.y, chunk = blockIdx.x, t = threadIdx.x;
  hist[t] = 0;
  __syncthreads();
  const int32_t* kh = keys + size_t(h) * N;
  const int base = chunk * SORT_CHUNK;
  for (int i = t; i < SORT_CHUNK; i += 256) {
    int n = base + i;
    if (n < N) atomicAdd(&hist[(kh[n] >> shift) & 255], 1);
  }
  __syncthreads();
  chist[(size_t(h) * 256 + t) * nchunks + chunk] = hist[t];
}

// exclusive scan of len ints per head (one workgroup of 1024 threads per head)
__global__ __launch_bounds__(1024) void scan_rows(const int32_t* __restrict__ in, int32_t* __restrict__ out,
                                                  int len, int out_stride, bool write_total) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int h = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int32_t* ih = in + size_t(h) * len;
  int32_t* oh = out + size_t(h) * out_stride;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int b = 0; b < len; b += 1024) {
    int i = b + t;
    int v = i < len ? ih[i] : 0;
    // inclusive wave scan
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int pre = carry_s;
    for (int j = 0; j < w; ++j) pre += wsum[j];
    if (i < len) oh[i] = pre + x - v;
    __syncthreads();
    if (t == 1023) carry_s = pre + x;
    __syncthreads();
  }
  if (write_total && t == 0) oh[len] = carry_s;
}

// stable scatter of one radix pass
__global__ __launch_bounds__(256) void sort_scatter(const int32_t* __restrict__ keys_in,
                                                    const int32_t* __restrict__ vals_in,
                                                    int32_t* __restrict__ keys_out,
                                                    int32_t* __restrict__ vals_out, int N, int shift,
                                                    int nchunks, const int32_t* __restrict__ cbase) {
  __shared__ int run[256];
  __shared__ int wc[4][256];
  const int h = blockIdx.y, chunk = blockIdx.x, t = threadIdx.x, w = t >> 6;
  run[t] = cbase[(size_t(h) * 256 + t) * nchunks + chunk];
  for (int j = 0; j < 4; ++j) wc[j][t] = 0;
  __syncthreads();
  const size_t hoff = size_t(h) * N;
  const int base = chunk * SORT_CHUNK;
  for (int r = 0; r < SORT_CHUNK; r += 256) {
    const int n = base + r + t;
    const bool valid = n < N;
    const int key = valid ? keys_in[hoff + n] : 0;
    const int val = valid ? (vals_in ? vals_in[hoff + n] : n) : 0;
    const int dig = (key >> shift) & 255;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < 8; ++b) {
      uint64_t bal = __ballot(valid && ((dig >> b) & 1));
      m &= ((dig >> b) & 1) ? bal : ~bal;
    }
    const int rank = __popcll(m & lanemask_lt());
    if (valid && rank == 0) wc[w][dig] = __popcll(m);
    __syncthreads();
    if (valid) {
      int pos = run[dig] + rank;
      for (int j = 0; j < w; ++j) pos += wc[j][dig];
      if (keys_out) keys_out[hoff + pos] = key;
      vals_out[hoff + pos] = val;
    }
    __syncthreads();
    run[t] += wc[0][t] + wc[1][t] + wc[2][t] + wc[3][t];
    wc[0][t] = wc[1][t] = wc[2][t] = wc[3][t] = 0;
    __syncthreads();
  }
}

__global__ void fill_i32(int32_t* p, size_t n, int32_t v) {
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Cluster sizes.  Few clusters: per-block LDS histograms of COUNT_CHUNK labels,
// then one global add per non-empty bin; many clusters: one global add per
// token (the adds spread over many addresses).  Integer adds: the result does
// not depend on their order.
constexpr int COUNT_CHUNK = 4096;
constexpr int COUNT_LDS_MAX = 4096;

__global__ __launch_bounds__(256) void count_labels_lds(const int32_t* __restrict__ labels, int N, int C,
                                                        int32_t* __restrict__ cnt) {
  __shared__ int hist[COUNT_LDS_MAX];
  const int h = blockIdx.y, t = threadIdx.x;
  for (int c = t; c < C; c += 256) hist[c] = 0;
  __syncthreads();
  const int a = blockIdx.x * COUNT_CHUNK, b = min(N, a + COUNT_CHUNK);
  const int32_t* lh = labels + size_t(h) * N;
  for (int n = a + t; n < b; n += 256) atomicAdd(&hist[lh[n]], 1);
  __syncthreads();
  for (int c = t; c < C; c += 256)
    if (hist[c]) atomicAdd(&cnt[size_t(h) * C + c], hist[c]);
}

__global__ __launch_bounds__(256) void count_labels(const int32_t* __restrict__ labels, int N, int C,
                                                    int32_t* __restrict__ cnt) {
  const int h = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n < N) atomicAdd(&cnt[size_t(h) * C + labels[size_t(h) * N + n]], 1);
}

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x, T* __restrict__ xp,
                                                     const int32_t* __restrict__ perm, int N,
                                                     int vec_per_row) {
  // 16-byte vectors
  const int h = blockIdx.y;
  const size_t g = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = size_t(N) * vec_per_row;
  if (g >= total) return;
  const int p = int(g / vec_per_row), c = int(g % vec_per_row);
  const int src = perm[size_t(h) * N + p];
  const uint4* s = reinterpret_cast<const uint4*>(x) + (size_t(h) * N + src) * vec_per_row + c;
  uint4* dst = reinterpret_cast<uint4*>(xp) + (size_t(h) * N + p) * vec_per_row + c;
  *dst = *s;
}

// Member means in two launches.  means_part_kernel: workgroup (c S + s, h)
// sums slice s of cluster c's rows (the cluster's rows cut into S equal
// runs); each thread owns one 16-byte vector (EPV elements) of the row slice
// [col0, col0 + dc) and sums its rows r, r + RPI, r + 2 RPI, ... of the run in
// that order (four loads in flight); the RPI partial sums of a column are then
// added in row-group order.  means_combine_kernel adds the S run sums in run
// order and divides by the cluster size.  The result is independent of timing.
template <typename T>
__global__ __launch_bounds__(256) void means_part_kernel(const T* __restrict__ x, int d, int col0, int dc,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ off, int N, int C, int S,
                                                         float* __restrict__ part_out) {
  constexpr int EPV = 16 / sizeof(T);
  __shared__ float part[256 * EPV];
  const int c = blockIdx.x / S, sl = blockIdx.x % S, h = blockIdx.y, t = threadIdx.x;
  const int ca = off[size_t(h) * (C + 1) + c], cb = off[size_t(h) * (C + 1) + c + 1];
  const int len = ceil_div(cb - ca, S);
  const int a = min(cb, ca + sl * len), b = min(cb, a + len);
  float* o = part_out + ((size_t(h) * C + c) * S + sl) * dc;
  const int V = dc / EPV;          // vectors per row slice
  const int RPI = 256 / V;         // rows per iteration
  const int r = t / V, j = t % V;
  const bool act = r < RPI;
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
  const int32_t* ph = perm + size_t(h) * N;
  const T* xh = x + size_t(h) * N * d + col0 + j * EPV;
  if (act) {
    constexpr int U = 4;
    for (int p0 = a + r; p0 < b; p0 += U * RPI) {
      uint4 raw[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int p = p0 + q * RPI;
        raw[q] = p < b ? *reinterpret_cast<const uint4*>(xh + size_t(ph[p]) * d) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        if (p0 + q * RPI >= b) break;
        if constexpr (sizeof(T) == 4) {
          acc[0] += __uint_as_float(raw[q].x);
          acc[1] += __uint_as_float(raw[q].y);
          acc[2] += __uint_as_float(raw[q].z);
          acc[3] += __uint_as_float(raw[q].w);
        } else {
          const uint32_t w4[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[2 * k] += __uint_as_float(w4[k] << 16);
            acc[2 * k + 1] += __uint_as_float(w4[k] & 0xFFFF0000u);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) part[r * dc + j * EPV + e] = acc[e];
  }
  __syncthreads();
  if (t < dc) {
    const int rows = min(RPI, b - a);
    float sum = 0.f;
    for (int k = 0; k < rows; ++k) sum += part[k * dc + t];
    o[t] = sum;
  }
}

__global__ __launch_bounds__(256) void means_combine_kernel(const float* __restrict__ part_in,
                                                            const int32_t* __restrict__ off, int C, int S,
                                                            int dc, float* __restrict__ out, int out_stride,
                                                            bool keep_empty) {
  const int c = blockIdx.x, h = blockIdx.y;
  const int n = off[size_t(h) * (C + 1) + c + 1] - off[size_t(h) * (C + 1) + c];
  float* o = out + (size_t(h) * C + c) * out_stride;
  const float* pi = part_in + (size_t(h) * C + c) * S * dc;
  for (int t = threadIdx.x; t < dc; t += blockDim.x) {
    if (n == 0) {
      if (!keep_empty) o[t] = 0.f;
      continue;
    }
    float sum = 0.f;
    for (int sl = 0; sl < S; ++sl) sum += pi[sl * dc + t];
    o[t] = sum / float(n);
  }
}

// Rows into cluster order and member means in one pass: one workgroup per
// (cluster, head) copies its rows to their cluster-order positions and sums
// them in the order of means_part_kernel with a single run (thread (r, j)
// takes rows r, r + RPI, ...; the RPI partial sums are added in row-group
// order).  An empty cluster's mean is zero.
template <typename T>
__global__ __launch_bounds__(256) void gather_means_kernel(const T* __restrict__ x, T* __restrict__ xp,
                                                           const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ off, int N, int C,
                                                           int d, float* __restrict__ out) {
  constexpr int EPV = 16 / sizeof(T);
  __shared__ float part[256 * EPV];
  const int c = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int a = off[size_t(h) * (C + 1) + c], b = off[size_t(h) * (C + 1) + c + 1];
  float* o = out + (size_t(h) * C + c) * d;
  if (b == a) {
    for (int j = t; j < d; j += 256) o[j] = 0.f;
    return;
  }
  const int V = d / EPV;   // vectors per row
  const int RPI = 256 / V; // rows per iteration
  const int r = t / V, j = t % V;
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
  const int32_t* ph = perm + size_t(h) * N;
  const uint4* xh = reinterpret_cast<const uint4*>(x + size_t(h) * N * d) + j;
  uint4* yh = reinterpret_cast<uint4*>(xp + size_t(h) * N * d) + j;
  constexpr int U = 4;
  for (int p0 = a + r; p0 < b; p0 += U * RPI) {
    uint4 raw[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int p = p0 + q * RPI;
      raw[q] = p < b ? xh[size_t(ph[p]) * V] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int p = p0 + q * RPI;
      if (p >= b) break;
      yh[size_t(p) * V] = raw[q];
      if constexpr (sizeof(T) == 4) {
        acc[0] += __uint_as_float(raw[q].x);
        acc[1] += __uint_as_float(raw[q].y);
        acc[2] += __uint_as_float(raw[q].z);
        acc[3] += __uint_as_float(raw[q].w);
      } else {
        const uint32_t w4[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += __uint_as_float(w4[k] << 16);
          acc[2 * k + 1] += __uint_as_float(w4[k] & 0xFFFF0000u);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPV; ++e) part[r * d + j * EPV + e] = acc[e];
  __syncthreads();
  if (t < d) {
    const int rows = min(RPI, b - a);
    float sum = 0.f;
    for (int k = 0; k < rows; ++k) sum += part[k * d + t];
    o[t] = sum / float(b - a);
  }
}

__global__ void raster_label_kernel(int32_t* __restrict__ labels, int N, int height, int width, int bt, int bh,
                                    int bw, int nh, int nw) {
  const int h = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int w = n % width, r = n / width, y = r % height, t = r / height;
  labels[size_t(h) * N + n] = ((t / bt) * nh + y / bh) * nw + w / bw;
}

__global__ __launch_bounds__(256) void labels_from_off_kernel(const int32_t* __restrict__ perm,
                                                              const int32_t* __restrict__ off,
                                                              int32_t* __restrict__ labels, int N,
                                                              int C) {
  const int c = blockIdx.x, h = blockIdx.y;
  const int a = off[size_t(h) * (C + 1) + c], b = off[size_t(h) * (C + 1) + c + 1];
  for (int p = a + threadIdx.x; p < b; p += 256)
    labels[size_t(h) * N + perm[size_t(h) * N + p]] = c;
}

}  // namespace

size_t label_sort_scratch(int H, int N, int C) {
  const int nchunks = ceil_div(N, SORT_CHUNK);
  Arena a{nullptr, 0, 0};
  a.get<int32_t>(size_t(H) * 256 * nchunks);  // chist
  a.get<int32_t>(size_t(H) * 256 * nchunks);  // cbase
  a.get<int32_t>(size_t(H) * N);              // tmp keys
  a.get<int32_t>(size_t(H) * N);              // tmp vals
  a.get<int32_t>(size_t(H) * C);              // counts
  return a.used;
}

hipError_t label_sort(const int32_t* labels, int32_t* perm, int32_t* offsets, int H, int N, int C,
                      Arena& s, hipStream_t st) {
  const int nchunks = ceil_div(N, SORT_CHUNK);
  int32_t* chist = s.get<int32_t>(size_t(H) * 256 * nchunks);
  int32_t* cbase = s.get<int32_t>(size_t(H) * 256 * nchunks);
  int32_t* tk = s.get<int32_t>(size_t(H) * N);
  int32_t* tv = s.get<int32_t>(size_t(H) * N);
  int32_t* cnt = s.get<int32_t>(size_t(H) * C);
  const int passes = C <= 256 ? 1 : (C <= 65536 ? 2 : 0);
  if (!passes) return hipErrorInvalidValue;
  dim3 g(nchunks, H);
  for (int ps = 0; ps < passes; ++ps) {
    const int shift = 8 * ps;
    const int32_t* kin = ps == 0 ? labels : tk;
    const int32_t* vin = ps == 0 ? nullptr : tv;
    const bool last = ps == passes - 1;
    sort_hist<<<g, 256, 0, st>>>(kin, N, shift, nchunks, chist);
    scan_rows<<<H, 1024, 0, st>>>(chist, cbase, 256 * nchunks, 256 * nchunks, false);
    // pass 0 of 2 writes to tmp, the last pass writes perm (keys not needed)
    if (passes == 2 && ps == 0) {
      sort_scatter<<<g, 256, 0, st>>>(kin, vin, tk, tv, N, shift, nchunks, cbase);
    } else {
      // in-place hazard: pass 1 reads tk/tv and writes perm only
      sort_scatter<<<g, 256, 0, st>>>(kin, vin, nullptr, perm, N, shift, nchunks, cbase);
    }
    (void)last;
  }
  // offsets from label counts
  size_t nc = size_t(H) * C;
  fill_i32<<<ceil_div(int(nc), 256), 256, 0, st>>>(cnt, nc, 0);
  if (C <= COUNT_LDS_MAX)
    count_labels_lds<<<dim3(ceil_div(N, COUNT_CHUNK), H), 256, 0, st>>>(labels, N, C, cnt);
  else
    count_labels<<<dim3(ceil_div(N, 256), H), 256, 0, st>>>(labels, N, C, cnt);
  scan_rows<<<H, 1024, 0, st>>>(cnt, offsets, C, C + 1, true);
  return hipGetLastError();
}

hipError_t gather_rows(const void* x, void* x_perm, const int32_t* perm, int H, int N, int d,
                       int dtype, hipStream_t st) {
  const int esz = dtype == SA_F32 ? 4 : 2;
  const int vpr = d * esz / 16;
  const size_t total = size_t(N) * vpr;
  dim3 g(unsigned((total + 255) / 256), H);
  gather_kernel<uint4><<<g, 256, 0, st>>>(reinterpret_cast<const uint4*>(x),
                                          reinterpret_cast<uint4*>(x_perm), perm, N, vpr);
  return hipGetLastError();
}

int means_runs(int H, int N, int C) {
  // enough workgroups to fill the chip (about 4096), runs of at least 32 rows
  const int want = ceil_div(4096, max(1, C * H));
  const int cap = max(1, N / max(1, C * 32));
  return max(1, min(16, min(want, cap)));
}

size_t means_scratch(int H, int N, int C, int dc) {
  return size_t(H) * C * means_runs(H, N, C) * dc * sizeof(float);
}

hipError_t cluster_means(const void* x, int dtype, int d, int col0, int dc, const int32_t* perm,
                         const int32_t* offsets, int H, int N, int C, float* out, int out_stride,
                         bool keep_empty, float* scratch, hipStream_t st) {
  const int esz = dtype == SA_F32 ? 4 : 2;
  // 16-byte vectors of the slice; at most 256 of them per row
  if ((col0 * esz) % 16 || (dc * esz) % 16 || (d * esz) % 16 || dc * esz > 256 * 16) return hipErrorInvalidValue;
  const int S = means_runs(H, N, C);
  dim3 g(C * S, H);
  if (dtype == SA_F32)
    means_part_kernel<float><<<g, 256, 0, st>>>((const float*)x, d, col0, dc, perm, offsets, N, C, S, scratch);
  else
    means_part_kernel<bf16_t><<<g, 256, 0, st>>>((const bf16_t*)x, d, col0, dc, perm, offsets, N, C, S, scratch);
  means_combine_kernel<<<dim3(C, H), 128, 0, st>>>(scratch, offsets, C, S, dc, out, out_stride, keep_empty);
  return hipGetLastError();
}

hipError_t gather_means(const void* x, int dtype, int d, const int32_t* perm, const int32_t* offsets,
                        int H, int N, int C, void* x_perm, float* means, hipStream_t st) {
  const int esz = dtype == SA_F32 ? 4 : 2;
  // 16-byte vectors, at most 256 of them per row
  if ((d * esz) % 16 || d * esz > 256 * 16) return hipErrorInvalidValue;
  dim3 g(C, H);
  if (dtype == SA_F32)
    gather_means_kernel<float><<<g, 256, 0, st>>>((const float*)x, (float*)x_perm, perm, offsets, N, C, d, means);
  else
    gather_means_kernel<bf16_t><<<g, 256, 0, st>>>((const bf16_t*)x, (bf16_t*)x_perm, perm, offsets, N, C, d,
                                                   means);
  return hipGetLastError();
}

hipError_t raster_labels(int32_t* labels, int H, int frames, int height, int width, const int* ext,
                         hipStream_t st) {
  const int N = frames * height * width;
  raster_label_kernel<<<dim3(ceil_div(N, 256), H), 256, 0, st>>>(labels, N, height, width, ext[0], ext[1], ext[2],
                                                                 ceil_div(height, ext[1]), ceil_div(width, ext[2]));
  return hipGetLastError();
}

hipError_t labels_from_offsets(const int32_t* perm, const int32_t* offsets, int32_t* labels, int H,
                               int N, int C, hipStream_t st) {
  labels_from_off_kernel<<<dim3(C, H), 256, 0, st>>>(perm, offsets, labels, N, C);
  return hipGetLastError();
}

}  // namespace sa
