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

// --------------------------------------------------------------------------
// SCOPE subspace keys: lookup-table scores over combos, selection in keys
// --------------------------------------------------------------------------
// SCOPE (technical framework, key design): T_s[i][c] = <qbar_i|_s, kbar^s_c>
// scale for each of the t/h/w slices; a combo g = (a_t, a_h, a_w) scores
// T_t[a_t] + T_h[a_h] + T_w[a_w] (+ ln|g|), and the selection counts keys.
// Rank order is (logit descending, combo ascending); the boundary of every
// cumulative target (mass, floor keys, online Top-k keys) is found by an exact
// weighted radix search over 64-bit order keys, masses in 2^-52 fixed point
// so their sums are exact and order independent.
constexpr int SUB_T = 1024;
constexpr double MASS_ONE = 4503599627370496.0;  // 2^52

struct SubRow {
  double T[3][32];
  unsigned long long hw[2048];   // radix bin weights (mass or keys)
  unsigned long long wsum[16];
  unsigned long long red[2][16];
  double dred[16];
  uint32_t words[1024];
  int sel_bin;
  unsigned long long sel_w;
  int tie_g;
};

__device__ __forceinline__ unsigned long long order_key(double l) {
  // ascending order of the key = descending logit
  unsigned long long u = __double_as_longlong(l + 0.0);
  u = (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
  return ~u;
}

// A position in rank order: every combo with a smaller order key, or the same
// key and g' <= g, lies at or before it.  g = -1: before every combo; g = C:
// past every combo.
struct Boundary {
  unsigned long long key;
  int g;
};

__device__ __forceinline__ bool before_or_at(unsigned long long k, int g, const Boundary& b) {
  return k < b.key || (k == b.key && g <= b.g);
}

template <typename V>
__device__ V bscan(V v, V* wsum, V& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
  V x = v;
  for (int o = 1; o < 64; o <<= 1) {
    V y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  V pre = 0, tot = 0;
  for (int j = 0; j < nw; ++j) {
    if (j < w) pre += wsum[j];
    tot += wsum[j];
  }
  total = tot;
  __syncthreads();
  return pre + x - v;
}

// First combo (in rank order) at which the cumulative weight reaches `target`
// (WK = 0: mass, 1: keys); g = C when the total stays below the target.
// Radix rounds of up to 11 bits narrow the order key from the top; combos
// sharing the final key are then taken in ascending g.
template <int WK, typename Eval>
__device__ Boundary wselect(Eval ev, int C, unsigned long long target, unsigned long long kmin,
                            unsigned long long kmax, SubRow& R) {
  const int t = threadIdx.x;
  unsigned long long prefix = kmin, rem = target;
  int hb = kmin == kmax ? -1 : 63 - __clzll(kmin ^ kmax);
  if (hb >= 0) prefix = hb == 63 ? 0ull : (kmin & ~((2ull << hb) - 1ull));
  while (hb >= 0) {
    const int shift = max(hb - 10, 0);
    const int width = hb - shift + 1;
    const unsigned long long dmask = (1ull << width) - 1ull;
    const int above = shift + width;
    for (int b = t; b < 2048; b += SUB_T) R.hw[b] = 0ull;
    __syncthreads();
    for (int g = t; g < C; g += SUB_T) {
      unsigned long long k, mass, keys;
      if (!ev(g, k, mass, keys)) continue;
      if (above < 64 && (k >> above) != (prefix >> above)) continue;
      atomicAdd(&R.hw[int((k >> shift) & dmask)], WK == 0 ? mass : keys);
    }
    __syncthreads();
    const unsigned long long w0 = R.hw[2 * t], w1 = R.hw[2 * t + 1];
    unsigned long long tw;
    const unsigned long long pw = bscan<unsigned long long>(w0 + w1, R.wsum, tw);
    if (t == 0) R.sel_bin = -1;
    __syncthreads();
    if (pw < rem && rem <= pw + w0) {
      R.sel_bin = 2 * t;
      R.sel_w = pw;
    } else if (pw + w0 < rem && rem <= pw + w0 + w1) {
      R.sel_bin = 2 * t + 1;
      R.sel_w = pw + w0;
    }
    __syncthreads();
    const int sb = R.sel_bin;
    const unsigned long long sw = R.sel_w;
    __syncthreads();
    if (sb < 0) return Boundary{0ull, C};  // target beyond the total: everything
    rem -= sw;
    prefix |= (unsigned long long)sb << shift;
    if (shift == 0) break;
    hb = shift - 1;
  }
  // ties on the order key: combos in ascending order
  unsigned long long run = 0;
  if (t == 0) R.tie_g = -1;
  __syncthreads();
  int tg = -1;
  for (int base = 0; base < C; base += SUB_T) {
    const int g = base + t;
    unsigned long long k = 0, mass = 0, keys = 0;
    const bool f = g < C && ev(g, k, mass, keys) && k == prefix;
    const unsigned long long wv = f ? (WK == 0 ? mass : keys) : 0ull;
    unsigned long long tot;
    const unsigned long long pre = bscan<unsigned long long>(wv, R.wsum, tot);
    if (f && run + pre < rem && rem <= run + pre + wv) R.tie_g = g;
    __syncthreads();
    tg = R.tie_g;
    __syncthreads();
    if (tg >= 0) break;
    run += tot;
  }
  // the total weight of the key reaches rem, so a combo is always found
  return Boundary{prefix, tg};
}

__device__ __forceinline__ bool later(const Boundary& a, const Boundary& b, int C) {
  // is boundary a later in rank order than b (C = past every combo)?
  if (a.g == C) return b.g != C;
  if (b.g == C) return false;
  return a.key > b.key || (a.key == b.key && a.g > b.g);
}

__global__ void logsize_kernel(const int32_t* __restrict__ k_off, int C, double* __restrict__ lg) {
  const int h = blockIdx.y;
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= C) return;
  const int sz = k_off[size_t(h) * (C + 1) + g + 1] - k_off[size_t(h) * (C + 1) + g];
  lg[size_t(h) * C + g] = sz > 0 ? log(double(sz)) : -__builtin_huge_val();
}

__global__ __launch_bounds__(SUB_T) void select_subspace(SelectArgs a, const double* __restrict__ lgs,
                                                         unsigned long long* __restrict__ acc,
                                                         int pass) {
  __shared__ SubRow R;
  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int Cq = a.Cq, C = a.Ck, Cs = a.Cs, d = a.d;
  const int W = ceil_div(C, 32);
  const size_t row = size_t(h) * Cq + i;
  const int32_t* qo = a.q_off + size_t(h) * (Cq + 1);
  const int qsize = qo[i + 1] - qo[i];
  const bool online = a.online != 0;
  if (qsize == 0) {
    if (!online || pass == 1) {
      for (int x = t; x < W; x += SUB_T) a.mask[row * W + x] = 0u;
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
  // lookup tables
  if (t < 3 * Cs) {
    const int sl = t / Cs, c = t % Cs;
    const int off = sl == 0 ? 0 : (sl == 1 ? a.dims[0] : a.dims[0] + a.dims[1]);
    const float* qb = a.qbar + row * d;
    const float* cb = a.kbar + (size_t(h) * 3 * Cs + sl * Cs + c) * d;
    double sdot = 0.0;
    for (int col = off; col < off + a.dims[sl]; ++col) sdot = fma(double(qb[col]), double(cb[col]), sdot);
    R.T[sl][c] = sdot * a.scale;
  }
  __syncthreads();
  const int32_t* ko = a.k_off + size_t(h) * (C + 1);
  const double* lh = lgs + size_t(h) * C;
  const int Cs2 = Cs * Cs;
  auto logit = [&](int g, double& l) -> bool {
    const double ls = lh[g];
    if (ls == -__builtin_huge_val()) return false;
    l = (R.T[0][g / Cs2] + R.T[1][(g / Cs) % Cs]) + R.T[2][g % Cs];
    if (a.weighted) l += ls;
    return true;
  };
  // max logit, normaliser, order-key range
  double mx = -__builtin_huge_val(), mn = __builtin_huge_val();
  for (int g = t; g < C; g += SUB_T) {
    double l;
    if (logit(g, l)) {
      mx = fmax(mx, l);
      mn = fmin(mn, l);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    mx = fmax(mx, __shfl_xor(mx, o, 64));
    mn = fmin(mn, __shfl_xor(mn, o, 64));
  }
  if (lane == 0) {
    R.red[0][w] = __double_as_longlong(mx);
    R.red[1][w] = __double_as_longlong(mn);
  }
  __syncthreads();
  mx = __longlong_as_double(R.red[0][0]);
  mn = __longlong_as_double(R.red[1][0]);
  for (int j = 1; j < SUB_T / 64; ++j) {
    mx = fmax(mx, __longlong_as_double(R.red[0][j]));
    mn = fmin(mn, __longlong_as_double(R.red[1][j]));
  }
  __syncthreads();
  double zs = 0.0;
  for (int g = t; g < C; g += SUB_T) {
    double l;
    if (logit(g, l)) zs += exp(l - mx);
  }
  for (int o = 32; o > 0; o >>= 1) zs += __shfl_xor(zs, o, 64);
  if (lane == 0) R.dred[w] = zs;
  __syncthreads();
  double Z = 0.0;
  for (int j = 0; j < SUB_T / 64; ++j) Z += R.dred[j];
  __syncthreads();
  const unsigned long long kmin = order_key(mx), kmax = order_key(mn);
  auto ev = [&](int g, unsigned long long& k, unsigned long long& mass, unsigned long long& keys) -> bool {
    double l;
    if (!logit(g, l)) return false;
    k = order_key(l);
    mass = (unsigned long long)llrint(exp(l - mx) / Z * MASS_ONE);
    keys = (unsigned long long)(ko[g + 1] - ko[g]);
    return true;
  };
  const int Cfull = C;
  const Boundary b0{0ull, -1};  // before every combo
  Boundary bp = b0, bf = b0;
  const double P = a.top_p;
  if (P >= 1.0) {
    bp = Boundary{0ull, Cfull};
  } else if (P > 0.0) {
    bp = wselect<0>(ev, C, (unsigned long long)llrint(P * MASS_ONE), kmin, kmax, R);
  }
  if (a.floor_units > 0) bf = wselect<1>(ev, C, (unsigned long long)a.floor_units, kmin, kmax, R);
  auto keys_through = [&](const Boundary& b) -> long long {
    // keys of every combo up to and including the boundary: the predicate
    // the mask is built from, so counts and mask agree by construction
    if (b.g < 0) return 0;
    unsigned long long sk = 0;
    for (int g = t; g < C; g += SUB_T) {
      double l;
      if (!logit(g, l)) continue;
      if (b.g == Cfull || before_or_at(order_key(l), g, b)) sk += (unsigned long long)(ko[g + 1] - ko[g]);
    }
    unsigned long long tot;
    bscan<unsigned long long>(sk, R.wsum, tot);
    return (long long)tot;
  };
  const Boundary binit = (bp.g < 0) ? bf : (bf.g < 0 ? bp : (later(bf, bp, Cfull) ? bf : bp));
  const long long n_init = keys_through(binit);
  if (online && pass == 0) {
    if (t == 0) {
      atomicAdd(&acc[h], (unsigned long long)((long long)qsize * n_init));
      if (a.init_counts) a.init_counts[row] = int(n_init);
    }
    return;
  }
  Boundary bfin = binit;
  int kh = 0;
  if (online) {
    const long long A = (long long)acc[h];
    kh = int((A + a.N - 1) / a.N);
    if (n_init < kh) {
      const Boundary bk = wselect<1>(ev, C, (unsigned long long)kh, kmin, kmax, R);
      if (binit.g < 0 || later(bk, binit, Cfull)) bfin = bk;
    }
  }
  const long long n_fin = keys_through(bfin);
  for (int x = t; x < W; x += SUB_T) R.words[x] = 0u;
  __syncthreads();
  if (bfin.g >= 0) {
    for (int g = t; g < C; g += SUB_T) {
      unsigned long long k, m2, ky;
      if (!ev(g, k, m2, ky)) continue;
      if (bfin.g == Cfull || before_or_at(k, g, bfin)) atomicOr(&R.words[g >> 5], 1u << (g & 31));
    }
  }
  __syncthreads();
  for (int x = t; x < W; x += SUB_T) a.mask[row * W + x] = R.words[x];
  if (t == 0) {
    a.counts[row] = int(n_fin);
    if (a.init_counts) a.init_counts[row] = int(n_init);
    if (i == 0) a.head_topk[h] = kh;
  }
}

}  // namespace

size_t select_scratch(int H, int Cq, int Ck, int subspace) {
  (void)Cq;
  Arena a{nullptr, 0, 0};
  a.get<unsigned long long>(size_t(H));
  if (subspace) a.get<double>(size_t(H) * Ck);
  return a.used;
}

hipError_t select_run(const SelectArgs& a, Arena& s, hipStream_t st) {
  unsigned long long* acc = s.get<unsigned long long>(size_t(a.H));
  dim3 g(a.Cq, a.H);
  if (a.subspace) {
    if (a.Cs > 32) return hipErrorInvalidValue;
    double* lgs = s.get<double>(size_t(a.H) * a.Ck);
    logsize_kernel<<<dim3(ceil_div(a.Ck, 256), a.H), 256, 0, st>>>(a.k_off, a.Ck, lgs);
    if (a.online) {
      zero_u64<<<ceil_div(a.H, 256), 256, 0, st>>>(acc, a.H);
      select_subspace<<<g, SUB_T, 0, st>>>(a, lgs, acc, 0);
      select_subspace<<<g, SUB_T, 0, st>>>(a, lgs, acc, 1);
    } else {
      select_subspace<<<g, SUB_T, 0, st>>>(a, lgs, acc, 0);
    }
    return hipGetLastError();
  }
  if (a.Ck > SEL_MAX || a.d > 128) return hipErrorInvalidValue;
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
