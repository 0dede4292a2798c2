// Centroid proxy scores and hybrid Top-p / fixed Top-k selection with SCOPE's
// online per-head Top-k (SCOPE, English abstract and key design section).
//
// One workgroup per (query cluster, head).  The row's proxy logits
//   l_j = <qbar_i, kbar_j> * scale (+ ln|K_j|),   empty key cluster -> excluded
// and its softmax are evaluated in fp64 (cheap at this size and accurate
// enough that the ranking and the Top-p crossing agree with an fp64 reference
// except at genuine ties).  The row is ranked by (p descending, j ascending)
// with an LDS bitonic sort; a block prefix sum of the masses gives the Top-p
// crossing.  The initial prefix is the shortest meeting both the mass and the
// floor.  With online Top-k, a first pass accumulates A_h = sum_i |Q_i| n_i
// with integer atomics (order independent, exact); the second pass computes
// k_h = ceil(A_h / n) and extends the rows below it along the same ranking.
// Every other reduction runs in a fixed order, so results are deterministic.

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int SEL_MAX = 1024;  // key clusters handled by the LDS sort

struct RowEntry {
  double p;
  int j;
};

__device__ __forceinline__ bool before(const RowEntry& a, const RowEntry& b) {
  return a.p > b.p || (a.p == b.p && a.j < b.j);
}

// block (256 threads) reductions in a fixed order
__device__ double block_max_d(double v, double* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3]));
}
__device__ double block_sum_d(double v, double* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}
__device__ int block_min_i(int v, int* sh) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return min(min(sh[0], sh[1]), min(sh[2], sh[3]));
}

__global__ void zero_u64(unsigned long long* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// pass 0: single pass (online off) or the first pass (online on, accumulate A_h)
// pass 1: second pass of online Top-k (extend and write)
__global__ __launch_bounds__(256) void select_rows(SelectArgs a, unsigned long long* __restrict__ acc,
                                                   int pass) {
  __shared__ RowEntry e[SEL_MAX];
  __shared__ double qd[128];
  __shared__ double red_d[4];
  __shared__ int red_i[4];
  __shared__ double tsum[256];
  __shared__ uint32_t words[SEL_MAX / 32];
  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int Cq = a.Cq, Ck = a.Ck, d = a.d;
  const int W = ceil_div(Ck, 32);
  const int32_t* qo = a.q_off + size_t(h) * (Cq + 1);
  const int qsize = qo[i + 1] - qo[i];
  const bool online = a.online != 0;
  const size_t row = size_t(h) * Cq + i;

  // empty query cluster: selects nothing (and adds nothing to A_h)
  if (qsize == 0) {
    if (!online || pass == 1) {
      for (int w = t; w < W; w += 256) a.mask[row * W + w] = 0u;
      if (t == 0) {
        a.counts[row] = 0;
        if (a.init_counts) a.init_counts[row] = 0;
        if (i == 0) a.head_topk[h] = online ? int(((long long)acc[h] + a.N - 1) / a.N) : 0;
      }
    } else if (t == 0 && a.init_counts) {
      a.init_counts[row] = 0;
    }
    return;
  }

  if (t < d) qd[t] = double(a.qbar[row * d + t]);
  int n2 = 2;
  while (n2 < Ck) n2 <<= 1;
  __syncthreads();

  // logits
  const int32_t* ko = a.k_off + size_t(h) * (Ck + 1);
  double lmax = -__builtin_huge_val();
  for (int j = t; j < n2; j += 256) {
    double l = -__builtin_huge_val();
    if (j < Ck) {
      const int sz = ko[j + 1] - ko[j];
      if (sz > 0) {
        const float* kb = a.kbar + (size_t(h) * Ck + j) * d;
        double s = 0.0;
        for (int c = 0; c < d; ++c) s = fma(qd[c], double(kb[c]), s);
        l = s * a.scale;
        if (a.weighted) l += log(double(sz));
      }
    }
    e[j].p = l;
    e[j].j = j;
    lmax = fmax(lmax, l);
  }
  lmax = block_max_d(lmax, red_d);
  double zs = 0.0;
  for (int j = t; j < n2; j += 256) {
    const double l = e[j].p;
    zs += (l == -__builtin_huge_val()) ? 0.0 : exp(l - lmax);
  }
  const double Z = block_sum_d(zs, red_d);
  for (int j = t; j < n2; j += 256) {
    const double l = e[j].p;
    e[j].p = (l == -__builtin_huge_val()) ? -1.0 : exp(l - lmax) / Z;
  }
  __syncthreads();

  // bitonic sort into rank order
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int x = t; x < n2; x += 256) {
        const int y = x ^ jj;
        if (y > x) {
          RowEntry A = e[x], B = e[y];
          const bool asc = (x & k) == 0;
          if (asc ? before(B, A) : before(A, B)) {
            e[x] = B;
            e[y] = A;
          }
        }
      }
      __syncthreads();
    }
  }

  // valid count, prefix masses (each thread owns a contiguous run of n2/256)
  const int per = (n2 + 255) / 256;
  const int r0 = t * per;
  double loc = 0.0;
  int nvalid = 0;
  for (int r = r0; r < min(r0 + per, n2); ++r) {
    if (e[r].p >= 0.0) {
      loc += e[r].p;
      ++nvalid;
    }
  }
  tsum[t] = loc;
  // exclusive scan of the per-thread sums in thread order
  __syncthreads();
  __shared__ double tpre[256];
  if (t == 0) {
    double run = 0.0;
    for (int u = 0; u < 256; ++u) {
      tpre[u] = run;
      run += tsum[u];
    }
  }
  // valid units: block sum of nvalid
  int nv = nvalid;
  for (int o = 32; o > 0; o >>= 1) nv += __shfl_xor(nv, o, 64);
  __syncthreads();
  if ((t & 63) == 0) red_i[t >> 6] = nv;
  __syncthreads();
  const int Vn = red_i[0] + red_i[1] + red_i[2] + red_i[3];

  int tp;
  const double P = a.top_p;
  if (P >= 1.0) {
    tp = Vn;
  } else if (P <= 0.0) {
    tp = 0;
  } else {
    int first = 0x7fffffff;
    double run = tpre[t];
    for (int r = r0; r < min(r0 + per, n2); ++r) {
      if (e[r].p >= 0.0) {
        run += e[r].p;
        if (run >= P && first == 0x7fffffff) first = r + 1;
      }
    }
    first = block_min_i(first, red_i);
    tp = first == 0x7fffffff ? Vn : first;
  }
  const int tf = a.floor_units > 0 ? min(a.floor_units, Vn) : 0;
  const int t_init = max(tp, tf);

  if (online && pass == 0) {
    if (t == 0) {
      atomicAdd(&acc[h], (unsigned long long)((long long)qsize * t_init));
      if (a.init_counts) a.init_counts[row] = t_init;
    }
    return;
  }
  int t_fin = t_init;
  int kh = 0;
  if (online) {
    const long long A = (long long)acc[h];
    kh = int((A + a.N - 1) / a.N);
    if (t_init < kh) t_fin = max(t_init, min(kh, Vn));
  }
  for (int w = t; w < W; w += 256) words[w] = 0u;
  __syncthreads();
  for (int r = t; r < t_fin; r += 256) atomicOr(&words[e[r].j >> 5], 1u << (e[r].j & 31));
  __syncthreads();
  for (int w = t; w < W; w += 256) a.mask[row * W + w] = words[w];
  if (t == 0) {
    a.counts[row] = t_fin;
    if (a.init_counts) a.init_counts[row] = t_init;
    if (i == 0) a.head_topk[h] = kh;
  }
}

}  // namespace

size_t select_scratch(int H, int Cq, int Ck, int subspace) {
  (void)Cq;
  (void)Ck;
  (void)subspace;
  Arena a{nullptr, 0, 0};
  a.get<unsigned long long>(size_t(H));
  return a.used;
}

hipError_t select_run(const SelectArgs& a, Arena& s, hipStream_t st) {
  if (a.subspace || a.Ck > SEL_MAX || a.d > 128) return hipErrorInvalidValue;
  unsigned long long* acc = s.get<unsigned long long>(size_t(a.H));
  dim3 g(a.Cq, a.H);
  if (a.online) {
    zero_u64<<<ceil_div(a.H, 256), 256, 0, st>>>(acc, a.H);
    select_rows<<<g, 256, 0, st>>>(a, acc, 0);
    select_rows<<<g, 256, 0, st>>>(a, acc, 1);
  } else {
    select_rows<<<g, 256, 0, st>>>(a, acc, 0);
  }
  return hipGetLastError();
}

}  // namespace sa
