// k-means assignment (and seeding) for query/key clustering and for SCOPE's
// per-subspace key clustering (SCOPE, technical framework: the t/h/w slices
// of the post-RoPE keys are clustered independently).
//
// bf16 rows (the common case) go to the matrix cores: ||c||^2 - 2 x.c with
// the centroids split into three bf16 terms, so the dot products are
// fp32-accurate.  Other rows (fp32, or slices that are not whole 16-column
// steps) evaluate sum_t (x_t - c_t)^2 directly in fp32 on the vector ALU, two
// operations per (token, centroid, dimension).  Ties go to the smallest
// centroid index in both.

#include "sa_internal.h"

#include <algorithm>

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

// bf16 rows: the same assignment on the matrix cores.  argmin_j ||x - c_j||^2
// = argmin_j (||c_j||^2 - 2 x.c_j).  x is exact in bf16; each centroid is split
// into three bf16 terms (c = hi + mid + lo, the residual below 2^-24 |c|), so
// the dot products are fp32-accurate, and the expansion's rounding stays far
// inside the near-tie scale 1e-5 (||x||^2 + ||c||^2).  S^T = C X^T per block of
// 32 centroids x 32 tokens on 32x32x16 bf16 MFMA: lane (col, hi) owns token col
// and centroids 8 (r / 4) + 4 hi + r % 4 (r = 0..15) of the block, walked in
// ascending order with a strict compare, and the two lanes of a token keep
// the smaller (distance, index).  Centroid rows sit in LDS with a pitch of
// DC + 8 elements, an odd number of 16-byte chunks, so the 32 rows a fragment
// read touches fall on distinct banks.
template <int DC>
constexpr int mfma_pitch() {
  return DC + 8;
}
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ floatx16 kmfma(bf16x8_t a, bf16x8_t b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <int DC>
__global__ __launch_bounds__(256) void assign_mfma_kernel(const bf16_t* __restrict__ x, int d, int col0,
                                                          int N, int C, const float* __restrict__ cent,
                                                          int32_t* __restrict__ labels) {
  constexpr int P = mfma_pitch<DC>();
  constexpr int KS = DC / 16;  // k-steps of 16 columns
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int CP = (C + 31) & ~31;
  bf16_t* ct = reinterpret_cast<bf16_t*>(smem);                  // [3][CP][P]
  float* cn = reinterpret_cast<float*>(smem + size_t(3) * CP * P * 2);  // [CP] ||c||^2
  const int h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int col = lane & 31, hi = lane >> 5;
  const float* ch = cent + size_t(h) * C * DC;
  for (int e = t; e < CP * DC; e += 256) {
    const int c = e / DC, k = e % DC;
    const float v = c < C ? ch[size_t(c) * DC + k] : 0.f;
    const bf16_t t0 = f2bf(v);
    const float r1 = v - bf2f(t0);
    const bf16_t t1 = f2bf(r1);
    const bf16_t t2 = f2bf(r1 - bf2f(t1));
    ct[size_t(c) * P + k] = t0;
    ct[size_t(CP + c) * P + k] = t1;
    ct[size_t(2 * CP + c) * P + k] = t2;
  }
  for (int c = t; c < CP; c += 256) {
    float sq = 0.f;
    if (c < C)
      for (int k = 0; k < DC; ++k) sq = fmaf(ch[size_t(c) * DC + k], ch[size_t(c) * DC + k], sq);
    cn[c] = sq;
  }
  __syncthreads();
  // each wave: two blocks of 32 tokens
#pragma unroll 1
  for (int b = 0; b < 2; ++b) {
    const int tok = blockIdx.x * 256 + (2 * w + b) * 32 + col;
    const bool valid = tok < N;
    const bf16_t* row = x + (size_t(h) * N + (valid ? tok : 0)) * d + col0;
    bf16x8_t xf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 u = *reinterpret_cast<const uint4*>(row + 16 * s + 8 * hi);
      if (!valid) u = make_uint4(0, 0, 0, 0);
      xf[s] = __builtin_bit_cast(bf16x8_t, u);
    }
    float best = __builtin_huge_valf();
    int bj = 0x7fffffff;
    for (int cb = 0; cb < CP; cb += 32) {
      floatx16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int term = 0; term < 3; ++term)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint4 u = *reinterpret_cast<const uint4*>(ct + size_t(term * CP + cb + col) * P + 16 * s + 8 * hi);
          acc = kmfma(__builtin_bit_cast(bf16x8_t, u), xf[s], acc);
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = cb + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float dv = cn[c] - 2.f * acc[r];
        if (c < C && dv < best) {
          best = dv;
          bj = c;
        }
      }
    }
    const float ob = __shfl_xor(best, 32, 64);
    const int oj = __shfl_xor(bj, 32, 64);
    if (ob < best || (ob == best && oj < bj)) bj = oj;
    if (valid && hi == 0) labels[size_t(h) * N + tok] = bj;
  }
}

// One Lloyd step for bf16 rows in one pass over them: the assignment as
// above but with the roles of registers and LDS swapped (each wave keeps the
// three terms of one 32-cluster block in registers and reads the staged token
// rows from LDS, so the per-step LDS traffic is the rows', not the
// centroids' once per wave; the per-token minimum is then taken over the
// blocks in ascending order), then every workgroup's sums of its tokens'
// slices per cluster, as
// onehot(labels)^T X on the same MFMA (bf16 products of x and 1 are exact,
// sums in fp32 in a fixed order), and its per-cluster counts.  A workgroup
// takes G groups of 128 tokens (one 32-token block per wave); each group's
// rows go to LDS, where the X^T operand is read with the LDS transpose read
// (ds_read_b64_tr_b16: lane i of each 16 receives element i % 4 of the pieces
// addressed by lanes i / 4 + 4 j, so 4 tokens x 4 column pieces give 4 tokens
// of one column per lane).  The waves share out the (32 clusters, 32 columns)
// blocks of the sums.  Workgroup partials are added in workgroup order by
// kmeans_combine_kernel, which keeps the previous centroid of an empty cluster.
// Rows are staged with chunk c of row r at c ^ xswz(r), which puts every 16-lane
// group of a transpose read on distinct banks (exhaustive search over XOR
// swizzles of the row bits).
template <int CPR>
__device__ __forceinline__ int xswz(int r) {
  if constexpr (CPR == 16) return (r & 7) << 1;
  else if constexpr (CPR == 8) return (r & 3) << 1;
  else return ((r >> 1) & 1) << 1;  // CPR == 4
}
typedef short v4i16k_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const bf16_t* p) {
  const v4i16k_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16k_t __attribute__((address_space(3)))*)p);
  return __builtin_bit_cast(uint2, r);
}
constexpr int KSTEP_TOK = 128;  // tokens per group
template <int DC>
constexpr int step_dcp() {
  return (DC + 31) & ~31;  // columns of the staged rows (zero padded)
}
template <int DC>
__global__ __launch_bounds__(256) void kmeans_step_kernel(const bf16_t* __restrict__ x, int d, int col0, int N,
                                                          int C, int G, const bf16_t* __restrict__ ctab,
                                                          const float* __restrict__ cnorm,
                                                          int32_t* __restrict__ labels, float* __restrict__ psum,
                                                          int32_t* __restrict__ pcnt, int32_t* __restrict__ rank) {
  constexpr int P = mfma_pitch<DC>();
  constexpr int KS = DC / 16;
  constexpr int DCP = step_dcp<DC>();
  constexpr int CPR = DCP / 8;      // 16-byte chunks of a staged row
  constexpr int NDB = DCP / 32;     // 32-column blocks of the sums
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int CP = (C + 31) & ~31;
  const int nb = CP / 32;  // 32-cluster blocks (1..4)
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);                // [128][DCP] the group's rows
  float* rv = reinterpret_cast<float*>(xs + KSTEP_TOK * DCP);  // [4][128] per-block minimum distance
  int* rj = reinterpret_cast<int*>(rv + 4 * KSTEP_TOK);        // [4][128] its cluster
  int* lab = rj + 4 * KSTEP_TOK;                               // [128]
  int* cnt = lab + KSTEP_TOK;                                  // [CP]
  const int h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int col = lane & 31, hi = lane >> 5;
  // this wave's cluster block, and its share of the group's four 32-token
  // blocks (the waves of one cluster block split them)
  const int cbw = w % nb;
  const int gi = w / nb, gs = (4 - cbw + nb - 1) / nb;
  // A operand of the distance: the three bf16 terms of cluster 32 cbw + col,
  // columns 16 s + 8 hi .. + 7, in registers for the whole step; the norms of
  // the 16 clusters whose distances the lane's D-layout elements hold
  bf16x8_t cf[3][KS];
  float cnv[16];
  {
    const bf16_t* tab = ctab + size_t(h) * 3 * CP * P;
#pragma unroll
    for (int term = 0; term < 3; ++term)
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        cf[term][s2] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(tab + size_t(term * CP + 32 * cbw + col) * P + 16 * s2 + 8 * hi));
#pragma unroll
    for (int r = 0; r < 16; ++r) cnv[r] = cnorm[size_t(h) * CP + 32 * cbw + 8 * (r >> 2) + 4 * hi + (r & 3)];
  }
  for (int c = t; c < CP; c += 256) cnt[c] = 0;
  // zero padding columns of the staged rows (never written afterwards)
  if constexpr (CPR > DC / 8) {
    constexpr int PADC = CPR - DC / 8;
    for (int e = t; e < KSTEP_TOK * PADC; e += 256) {
      const int r = e / PADC, c = DC / 8 + e % PADC;
      *reinterpret_cast<uint4*>(xs + r * DCP + ((c ^ xswz<CPR>(r)) << 3)) = make_uint4(0, 0, 0, 0);
    }
  }
  // this wave's (cluster block, column block) pairs of the sums
  const int npairs = (CP / 32) * NDB;
  floatx16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  // transpose-read offsets: rows 16 ks + 8 j + tr_row share tr_row's swizzle
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int tr_off[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int cc = 32 * db + tr_col;
    tr_off[db] = tr_row * DCP + (((cc >> 3) ^ xswz<CPR>(tr_row)) << 3) + (cc & 7);
  }
  const int ntile = (N + KSTEP_TOK - 1) / KSTEP_TOK;
  const int lr = 32 * w + col;  // the row this lane stages
  // the staged row's 16-byte pieces 2 s + hi (zeros past N)
  uint4 xf[KS];
  auto load_rows = [&](int tile) {
    const int tok = tile * KSTEP_TOK + lr;
    const bool valid = tok < N;
    const bf16_t* row = x + (size_t(h) * N + (valid ? tok : 0)) * d + col0;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      xf[s2] = *reinterpret_cast<const uint4*>(row + 16 * s2 + 8 * hi);
      if (!valid) xf[s2] = make_uint4(0, 0, 0, 0);
    }
  };
  if (int(blockIdx.x) * G < ntile) load_rows(int(blockIdx.x) * G);
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    const int tile = blockIdx.x * G + g;
    if (tile >= ntile) break;  // uniform across the workgroup
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      *reinterpret_cast<uint4*>(xs + lr * DCP + (((2 * s2 + hi) ^ xswz<CPR>(lr)) << 3)) = xf[s2];
    __syncthreads();  // the group's rows are staged
    // the next group's rows travel while this one is computed
    if (g + 1 < G && tile + 1 < ntile) load_rows(tile + 1);
    // distances ||c||^2 - 2 x.c of the wave's cluster block to its token
    // blocks (B operand: token rows from LDS), the three terms accumulated in
    // the same order as one centroid row at a time; per token the smallest,
    // first index on ties
#pragma unroll 1
    for (int tb = gi; tb < 4; tb += gs) {
      const int xr = 32 * tb + col;
      floatx16 a2;
#pragma unroll
      for (int r = 0; r < 16; ++r) a2[r] = 0.f;
#pragma unroll
      for (int term = 0; term < 3; ++term)
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const uint4 u = *reinterpret_cast<const uint4*>(xs + xr * DCP + (((2 * s2 + hi) ^ xswz<CPR>(xr)) << 3));
          a2 = kmfma(cf[term][s2], __builtin_bit_cast(bf16x8_t, u), a2);
        }
      float best = __builtin_huge_valf();
      int bj = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * cbw + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float dv = cnv[r] - 2.f * a2[r];
        if (c < C && dv < best) {
          best = dv;
          bj = c;
        }
      }
      const float ob = __shfl_xor(best, 32, 64);
      const int oj = __shfl_xor(bj, 32, 64);
      if (ob < best || (ob == best && oj < bj)) {
        best = ob;
        bj = oj;
      }
      if (hi == 0) {
        rv[cbw * KSTEP_TOK + xr] = best;
        rj[cbw * KSTEP_TOK + xr] = bj;
      }
    }
    __syncthreads();  // every block's minimum is in LDS
    if (t < KSTEP_TOK) {
      // blocks in ascending order, strict: the first index among equal minima
      float best = rv[t];
      int bj = rj[t];
      for (int cb = 1; cb < nb; ++cb) {
        const float v = rv[cb * KSTEP_TOK + t];
        if (v < best) {
          best = v;
          bj = rj[cb * KSTEP_TOK + t];
        }
      }
      const int tok = tile * KSTEP_TOK + t;
      const bool valid = tok < N;
      lab[t] = valid ? bj : -1;
      if (valid) {
        labels[size_t(h) * N + tok] = bj;
        if (!rank) atomicAdd(&cnt[bj], 1);
      }
    }
    __syncthreads();  // labels of the group are in LDS
    if (rank) {
      // each token's rank among the workgroup's tokens of its cluster, in
      // token order: the count before this group plus the group's earlier
      // tokens with the same label (a stable counting sort's position inside
      // the workgroup's share of the cluster)
      const int bj = t < KSTEP_TOK ? lab[t] : -1;
      if (bj >= 0) {
        int r = 0;
        for (int u = 0; u < t; ++u) r += lab[u] == bj ? 1 : 0;
        rank[size_t(h) * N + tile * KSTEP_TOK + t] = cnt[bj] + r;
      }
      __syncthreads();  // every count read before this group's are added
      if (bj >= 0) atomicAdd(&cnt[bj], 1);
    }
    // sums: for every 16-token step, the one-hot B operand from the labels of
    // the lane's 8 tokens (in the order the transpose reads give them)
#pragma unroll 1
    for (int ks = 0; ks < KSTEP_TOK / 16; ++ks) {
      int lv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lv[e] = lab[16 * ks + 4 * hi + e];
        lv[4 + e] = lab[16 * ks + 8 + 4 * hi + e];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pr = w + 4 * j;
        if (pr >= npairs) break;  // uniform across the wave
        const int cb = pr / NDB, db = pr % NDB;
        const int me = 32 * cb + col;
        uint32_t bw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bw[e] = (lv[2 * e] == me ? 0x3F80u : 0u) | (lv[2 * e + 1] == me ? 0x3F800000u : 0u);
        const uint2 v0 = lds_tr16(xs + tr_off[db] + (16 * ks) * DCP);
        const uint2 v1 = lds_tr16(xs + tr_off[db] + (16 * ks + 8) * DCP);
        acc[j] = kmfma(__builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y)),
                       __builtin_bit_cast(bf16x8_t, make_uint4(bw[0], bw[1], bw[2], bw[3])), acc[j]);
      }
    }
    __syncthreads();  // the next group overwrites the staged rows and labels
  }
  // partials: lane (col, hi) of pair (cb, db) holds the sums of cluster
  // 32 cb + col over columns 32 db + 8 (r / 4) + 4 hi + r % 4
  const size_t pb = size_t(h) * gridDim.x + blockIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pr = w + 4 * j;
    if (pr >= npairs) break;
    const int cb = pr / NDB, db = pr % NDB;
    float* dst = psum + (pb * CP + 32 * cb + col) * DC;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dim = 32 * db + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (dim < DC) dst[dim] = acc[j][r];
    }
  }
  for (int c = t; c < CP; c += 256) pcnt[pb * CP + c] = cnt[c];
}

// The centroid terms of the matrix-core distance for one centroid row (or a
// zero padding row when v is null): three bf16 terms hi + mid + lo of every
// column, at [term][CP][P] of the head's table, and the fp32 norm summed over
// the columns in ascending order.  One thread per column (DC <= 128 threads).
template <int DC>
__device__ __forceinline__ void write_ctab_row(const float* v, int c, int CP, bf16_t* tab, float* norm) {
  constexpr int P = mfma_pitch<DC>();
  const int k = threadIdx.x;
  const float x = v ? v[k] : 0.f;
  const bf16_t t0 = f2bf(x);
  const float r1 = x - bf2f(t0);
  const bf16_t t1 = f2bf(r1);
  const bf16_t t2 = f2bf(r1 - bf2f(t1));
  tab[size_t(c) * P + k] = t0;
  tab[size_t(CP + c) * P + k] = t1;
  tab[size_t(2 * CP + c) * P + k] = t2;
  if (k == 0) {
    float sq = 0.f;
    if (v)
      for (int j = 0; j < DC; ++j) sq = fmaf(v[j], v[j], sq);
    *norm = sq;
  }
}

// the table of every centroid row (padding rows zero) from fp32 centroids:
// before the first step of a run.  With sx (first-k seeding), the centroids
// are first set to the slice's first C rows of x, as seed_kernel would.
template <int DC>
__global__ __launch_bounds__(DC) void ctab_kernel(float* __restrict__ cent, int C, int CP,
                                                  bf16_t* __restrict__ ctab, float* __restrict__ cnorm,
                                                  const bf16_t* __restrict__ sx, int d, int col0, int N) {
  __shared__ float row[DC];
  const int c = blockIdx.x, h = blockIdx.y;
  if (c < C && sx) {
    const float v = bf2f(sx[(size_t(h) * N + c) * d + col0 + threadIdx.x]);
    cent[(size_t(h) * C + c) * DC + threadIdx.x] = v;
    row[threadIdx.x] = v;
  } else if (c < C) {
    row[threadIdx.x] = cent[(size_t(h) * C + c) * DC + threadIdx.x];
  }
  __syncthreads();
  write_ctab_row<DC>(c < C ? row : nullptr, c, CP, ctab + size_t(h) * 3 * CP * mfma_pitch<DC>(),
                     cnorm + size_t(h) * CP + c);
}

// centroid = (sum of the workgroup partials, in workgroup order) / count;
// an empty cluster keeps its centroid.  Also the next step's table row.
template <int DC>
__global__ __launch_bounds__(DC) void kmeans_combine_kernel(const float* __restrict__ psum,
                                                            const int32_t* __restrict__ pcnt, int nblk, int C,
                                                            int CP, float* __restrict__ cent,
                                                            bf16_t* __restrict__ ctab, float* __restrict__ cnorm) {
  __shared__ float row[DC];
  const int c = blockIdx.x, h = blockIdx.y, dim = threadIdx.x;
  float s2 = 0.f;
  long long n = 0;
  // eight partials in flight, added in workgroup order
  int b = 0;
  for (; b + 8 <= nblk; b += 8) {
    float v[8];
    int k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t pb = size_t(h) * nblk + b + u;
      v[u] = psum[(pb * CP + c) * DC + dim];
      k[u] = pcnt[pb * CP + c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s2 += v[u];
      n += k[u];
    }
  }
  for (; b < nblk; ++b) {
    const size_t pb = size_t(h) * nblk + b;
    s2 += psum[(pb * CP + c) * DC + dim];
    n += pcnt[pb * CP + c];
  }
  float* dst = cent + (size_t(h) * C + c) * DC + dim;
  const float v = n > 0 ? s2 / float(n) : *dst;
  if (n > 0) *dst = v;
  row[dim] = v;
  __syncthreads();
  write_ctab_row<DC>(row, c, CP, ctab + size_t(h) * 3 * CP * mfma_pitch<DC>(), cnorm + size_t(h) * CP + c);
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

// inverse of expand_kernel: the slice columns of each expanded row back into
// the compact blocks [3][H][Cs][d_s]
__global__ void compact_kernel(const float* __restrict__ in, int H, int Cs, int d, int d0, int d1, int d2,
                               float* __restrict__ sub) {
  const int h = blockIdx.y, row = blockIdx.x;  // row in [0, 3*Cs)
  const int s = row / Cs, c = row % Cs;
  const int ds[3] = {d0, d1, d2};
  const int off[3] = {0, d0, d0 + d1};
  size_t base = 0;
  for (int q = 0; q < s; ++q) base += size_t(H) * Cs * ds[q];
  float* dst = sub + base + (size_t(h) * Cs + c) * ds[s];
  const float* src = in + (size_t(h) * 3 * Cs + row) * d + off[s];
  for (int t = threadIdx.x; t < ds[s]; t += blockDim.x) dst[t] = src[t];
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

template <int DC>
hipError_t assign_mfma_launch(const void* x, int d, int col0, int H, int N, int C, const float* c,
                              int32_t* labels, hipStream_t st) {
  const int CP = (C + 31) & ~31;
  const size_t lds = size_t(3) * CP * mfma_pitch<DC>() * 2 + size_t(CP) * 4;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)assign_mfma_kernel<DC>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          int(lds)) != hipSuccess)
    return hipErrorInvalidValue;
  assign_mfma_kernel<DC><<<dim3(ceil_div(N, 256), H), 256, lds, st>>>((const bf16_t*)x, d, col0, N, C, c,
                                                                      labels);
  return hipGetLastError();
}

// The matrix-core path: bf16 rows whose 16-byte slices are aligned, widths
// that are whole 16-column steps, and up to 128 centroids (centroid terms in
// at most 105 KB of LDS).
bool assign_mfma_ok(const void* x, int d, int col0, int dc, int C) {
  return (reinterpret_cast<uintptr_t>(x) % 16 == 0) && d % 8 == 0 && col0 % 8 == 0 && dc % 16 == 0 &&
         C >= 1 && C <= 128;
}

template <typename T>
hipError_t assign_dispatch(const void* x, int d, int col0, int dc, int H, int N, int C,
                           const float* c, int32_t* labels, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (assign_mfma_ok(x, d, col0, dc, C)) {
      switch (dc) {
        case 16: return assign_mfma_launch<16>(x, d, col0, H, N, C, c, labels, st);
        case 32: return assign_mfma_launch<32>(x, d, col0, H, N, C, c, labels, st);
        case 48: return assign_mfma_launch<48>(x, d, col0, H, N, C, c, labels, st);
        case 64: return assign_mfma_launch<64>(x, d, col0, H, N, C, c, labels, st);
        case 128: return assign_mfma_launch<128>(x, d, col0, H, N, C, c, labels, st);
        default: break;
      }
    }
  }
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

// After the last fused step: the stable counting sort of the labels and the
// rows in cluster order, in one pass.  Workgroup (b, h) takes the tokens the
// step's workgroup b covered (whole groups of 128, in token order); a token
// of cluster c lands at offset[c] + (tokens of c in earlier workgroups) +
// its rank inside its workgroup, i.e. in (label, index) order.  Offsets come
// from the step's per-workgroup counts.  Cluster counts up to 128.
__global__ __launch_bounds__(256) void kmeans_scatter_kernel(const bf16_t* __restrict__ x, int d, int N, int C,
                                                             int CP, int nblk, int G,
                                                             const int32_t* __restrict__ pcnt,
                                                             const int32_t* __restrict__ labels,
                                                             const int32_t* __restrict__ rank,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ offsets,
                                                             bf16_t* __restrict__ x_perm) {
  __shared__ int base[128], tot[128], off[129];
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (t < CP) {
    int tb = 0, tt = 0;
    const int32_t* pc = pcnt + size_t(h) * nblk * CP + t;
    int bb = 0;
    for (; bb + 8 <= nblk; bb += 8) {  // eight counts in flight
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pc[size_t(bb + u) * CP];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (bb + u < b) tb += v[u];
        tt += v[u];
      }
    }
    for (; bb < nblk; ++bb) {
      const int v = pc[size_t(bb) * CP];
      if (bb < b) tb += v;
      tt += v;
    }
    base[t] = tb;
    tot[t] = tt;
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int c = 0; c < CP; ++c) {
      off[c] = run;
      run += tot[c];
    }
    off[CP] = run;
  }
  __syncthreads();
  if (b == 0)
    for (int c = t; c <= C; c += 256) offsets[size_t(h) * (C + 1) + c] = off[c];
  const int t0 = b * G * KSTEP_TOK, t1 = min(N, t0 + G * KSTEP_TOK);
  const size_t hn = size_t(h) * N;
  auto pos_of = [&](int tok) {
    const int c = labels[hn + tok];
    return off[c] + base[c] + rank[hn + tok];
  };
  for (int tok = t0 + t; tok < t1; tok += 256) perm[hn + pos_of(tok)] = tok;
  const int cpr = d / 8;  // 16-byte chunks of a row
  for (int v = t; v < (t1 - t0) * cpr; v += 256) {
    const int tok = t0 + v / cpr, ch = v % cpr;
    *reinterpret_cast<uint4*>(x_perm + (hn + pos_of(tok)) * d + ch * 8) =
        *reinterpret_cast<const uint4*>(x + (hn + tok) * d + ch * 8);
  }
}

// Workgroups per head of the fused step: about 1024 in all, but at most one
// per 2 CP tokens (so the partials, written and read once, move no more bytes
// than the rows), and whole groups of 128 tokens each.
void step_geometry(int H, int N, int C, int& nblk, int& G) {
  const int CP = (C + 31) & ~31;
  const int ntile = (N + KSTEP_TOK - 1) / KSTEP_TOK;
  int bh = std::max(1, std::min(ntile, (1024 + H - 1) / H));
  bh = std::max(1, std::min(bh, N / (2 * CP)));
  G = (ntile + bh - 1) / bh;
  nblk = (ntile + G - 1) / G;
}

// scratch of the fused step: partial sums [H][nblk][CP][DC] f32, counts
// [H][nblk][CP], then (256-byte aligned) the centroid table [H][3][CP][P]
// bf16 and norms [H][CP] f32
struct StepScratch {
  float* psum;
  int32_t* pcnt;
  bf16_t* ctab;
  float* cnorm;
  int32_t* rank;
  size_t bytes;
};
StepScratch step_scratch(int H, int N, int C, int dc, void* base) {
  int nblk, G;
  step_geometry(H, N, C, nblk, G);
  const size_t CP = size_t((C + 31) & ~31);
  const size_t P = size_t(dc) + 8;
  StepScratch r{};
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off = (off + b + 255) & ~size_t(255);
    return static_cast<char*>(base) + o;
  };
  r.psum = reinterpret_cast<float*>(take(size_t(H) * nblk * CP * dc * sizeof(float)));
  r.pcnt = reinterpret_cast<int32_t*>(take(size_t(H) * nblk * CP * sizeof(int32_t)));
  r.ctab = reinterpret_cast<bf16_t*>(take(size_t(H) * 3 * CP * P * sizeof(bf16_t)));
  r.cnorm = reinterpret_cast<float*>(take(size_t(H) * CP * sizeof(float)));
  r.rank = reinterpret_cast<int32_t*>(take(size_t(H) * N * sizeof(int32_t)));
  r.bytes = off;
  return r;
}

// Groups per workgroup for the launch: at least the G of step_geometry (which
// sizes the partials), and beyond it the G that minimises (rounds of
// workgroups over the chip) x G, with the kernel's real occupancy; ties go to
// the smaller G.  With one workgroup per CU, 344 workgroups of 2 groups take
// two rounds (4 group times) where 232 of 3 take one (3).
void launch_geometry(int H, int N, int C, int per_cu, int cus, int& nblk, int& G) {
  step_geometry(H, N, C, nblk, G);
  if (per_cu < 1 || cus < 1) return;
  const int ntile = (N + KSTEP_TOK - 1) / KSTEP_TOK;
  const long long slots = (long long)per_cu * cus;
  long long best = -1;
  int bestG = G;
  for (int g = G; g <= ntile; ++g) {
    const long long wgs = (long long)H * ((ntile + g - 1) / g);
    const long long cost = ((wgs + slots - 1) / slots) * g;
    if (best < 0 || cost < best) {
      best = cost;
      bestG = g;
    }
    if (wgs <= slots) break;  // one round: a larger G only adds group times
  }
  G = bestG;
  nblk = (ntile + G - 1) / G;
}

template <int DC>
hipError_t kmeans_step_launch(const void* x, int d, int col0, int H, int N, int C, float* c,
                              int32_t* labels, float* scratch, bool first, bool seed, const StepSort* sort,
                              hipStream_t st) {
  const int CP = (C + 31) & ~31;
  const StepScratch sc = step_scratch(H, N, C, DC, scratch);
  if (first)
    ctab_kernel<DC><<<dim3(CP, H), DC, 0, st>>>(c, C, CP, sc.ctab, sc.cnorm, seed ? (const bf16_t*)x : nullptr, d,
                                                col0, N);
  const size_t lds = size_t(KSTEP_TOK) * step_dcp<DC>() * 2 + size_t(9) * KSTEP_TOK * 4 + size_t(CP) * 4;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)kmeans_step_kernel<DC>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          int(lds)) != hipSuccess)
    return hipErrorInvalidValue;
  int per_cu = 0, cus = 0, dev = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kmeans_step_kernel<DC>, 256, lds) != hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    per_cu = cus = 0;  // the partials' geometry
  int nblk, G;
  launch_geometry(H, N, C, per_cu, cus, nblk, G);
  kmeans_step_kernel<DC><<<dim3(nblk, H), 256, lds, st>>>((const bf16_t*)x, d, col0, N, C, G, sc.ctab, sc.cnorm,
                                                          labels, sc.psum, sc.pcnt, sort ? sc.rank : nullptr);
  kmeans_combine_kernel<DC><<<dim3(C, H), DC, 0, st>>>(sc.psum, sc.pcnt, nblk, C, CP, c, sc.ctab, sc.cnorm);
  if (sort)
    kmeans_scatter_kernel<<<dim3(nblk, H), 256, 0, st>>>((const bf16_t*)x, d, N, C, CP, nblk, G, sc.pcnt, labels,
                                                        sc.rank, sort->perm, sort->offsets, (bf16_t*)sort->x_perm);
  return hipGetLastError();
}

}  // namespace

bool kmeans_step_supported(int dtype, const void* x, int d, int col0, int dc, int C) {
  return dtype == SA_BF16 && dc % 16 == 0 && dc <= 128 && assign_mfma_ok(x, d, col0, dc, C);
}

size_t kmeans_step_scratch(int H, int N, int C, int dc) {
  return step_scratch(H, N, C, dc, nullptr).bytes + 256;
}

hipError_t kmeans_step(const void* x, int d, int col0, int dc, int H, int N, int C, float* c,
                       int32_t* labels, float* scratch, bool first, bool seed, const StepSort* sort,
                       hipStream_t st) {
  // the fused sort covers whole rows only; seeding goes with the first step
  if ((sort && (col0 != 0 || dc != d)) || (seed && !first)) return hipErrorInvalidValue;
  switch (dc) {
    case 16: return kmeans_step_launch<16>(x, d, col0, H, N, C, c, labels, scratch, first, seed, sort, st);
    case 32: return kmeans_step_launch<32>(x, d, col0, H, N, C, c, labels, scratch, first, seed, sort, st);
    case 48: return kmeans_step_launch<48>(x, d, col0, H, N, C, c, labels, scratch, first, seed, sort, st);
    case 64: return kmeans_step_launch<64>(x, d, col0, H, N, C, c, labels, scratch, first, seed, sort, st);
    case 128: return kmeans_step_launch<128>(x, d, col0, H, N, C, c, labels, scratch, first, seed, sort, st);
    default: return hipErrorInvalidValue;
  }
}

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

hipError_t compact_sub_centroids(const float* expanded, int H, int Cs, int d, const int* dims, float* sub,
                                 hipStream_t st) {
  compact_kernel<<<dim3(3 * Cs, H), 128, 0, st>>>(expanded, H, Cs, d, dims[0], dims[1], dims[2], sub);
  return hipGetLastError();
}

}  // namespace sa
