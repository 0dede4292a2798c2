// Centroid proxy scores and hybrid Top-p / fixed Top-k selection with SCOPE's
// online per-head Top-k (SCOPE, English abstract and key design section).
//
// Proxy logits l_ij = <qbar_i, kbar_j> * scale (+ ln|K_j|) are evaluated in
// fp64 (an empty key cluster is excluded).  A row is ranked by (logit
// descending, j ascending); the boundary where a cumulative target is reached
// (softmax mass >= top_p, a count of units) is found by an exact weighted radix
// search over 64-bit order keys, with masses in 2^-52 fixed point so that
// their sums are exact and independent of order.  The initial prefix is the
// shortest meeting both the mass and the floor.  With online Top-k, a first
// pass accumulates A_h = sum_i |Q_i| n_i with integer atomics; the second
// computes k_h = ceil(A_h / n) and extends the rows below it along the same
// ranking.  Every other reduction runs in a fixed order: results are
// deterministic.
//
// Key clusters (KMEANS / BISECT): a tiled fp64 kernel forms every logit of a
// head, then one wavefront per query cluster selects.  SCOPE key subspaces:
// one workgroup per query cluster evaluates the 32^3 combo logits from the
// per-slice lookup tables on the fly; units are keys.

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int SEL_MAX = 1024;  // key clusters per row in cluster mode

__global__ void zero_u64(unsigned long long* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__global__ void fill_u64_kernel(unsigned long long* p, size_t n) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// pass 0: single pass (online off) or the first pass (online on, accumulate A_h)
// pass 1: second pass of online Top-k (extend and write)
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

constexpr int CAND = 1024;  // combos of the selected interpolated bin kept in LDS
constexpr int LOGT = 1024;  // ln(size) of combos smaller than this from an LDS table

struct SubRow {
  double T[3][32];
  unsigned long long hw[2048];   // radix bin weights (mass or keys)
  unsigned long long hk[2048];   // keys per interpolated bin (mass selection)
  unsigned long long wsum[16];
  unsigned long long red[2][16];
  double dred[16];
  double lt[LOGT];               // lt[s] = ln(s), lt[0] = -inf
  uint32_t words[1024];          // the row's mask, built by the selections
  uint16_t bin[32768];           // each combo's interpolated bin (0xffff: empty)
  unsigned long long ck[CAND];   // candidates: order key, weight, combo, keys
  unsigned long long cw[CAND];
  int cg[CAND];
  uint32_t ckeys[CAND];
  int ncand;
  int sel_bin;
  unsigned long long sel_w;
  unsigned long long sel_k;      // keys of the bins before the selected one
  int tie_g;
  unsigned long long tie_key;
  long long tie_keys;
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

// Every combo of the row, this thread's share, with sizes loaded four combos
// ahead of their use: f(g, size), size 0 for an empty combo.
constexpr int SUB_U = 4;
template <typename F>
__device__ __forceinline__ void for_combos(const int32_t* __restrict__ ksz, int C, F f) {
  for (int g = threadIdx.x; g < C; g += SUB_U * SUB_T) {
    int sz[SUB_U];
#pragma unroll
    for (int u = 0; u < SUB_U; ++u) sz[u] = g + u * SUB_T < C ? ksz[g + u * SUB_T] : 0;
#pragma unroll
    for (int u = 0; u < SUB_U; ++u)
      if (g + u * SUB_T < C) f(g + u * SUB_T, sz[u]);
  }
}
// The same with the wave kept together (for ballots): f(g0, size) for the
// lane's combo g0 + lane, size 0 past the end; g0 is the same in every lane.
template <typename F>
__device__ __forceinline__ void for_combo_waves(const int32_t* __restrict__ ksz, int C, F f) {
  const int lane = threadIdx.x & 63;
  for (int g0 = threadIdx.x - lane; g0 < C; g0 += SUB_U * SUB_T) {
    int sz[SUB_U];
#pragma unroll
    for (int u = 0; u < SUB_U; ++u) {
      const int g = g0 + u * SUB_T + lane;
      sz[u] = g < C ? ksz[g] : 0;
    }
#pragma unroll
    for (int u = 0; u < SUB_U; ++u)
      if (g0 + u * SUB_T < C) f(g0 + u * SUB_T, sz[u]);
  }
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

// The same boundary as wselect, with the keys of every combo at or before it,
// in two passes over the combos.  Pass 1 bins every combo by its logit,
// interpolated between the row's largest and smallest (bin = floor((mx - l)
// 2048 / (mx - mn)) is monotone in the logit, so the bins follow rank order),
// and finds the bin where the cumulative weight reaches the target.  Pass 2
// keeps that bin's combos in LDS; each counts the weight ranked before it,
// which names the boundary exactly.  ok = false when the bin holds more than
// CAND combos (the caller then runs wselect).
struct BoundK {
  Boundary b;
  long long keys;
  bool ok;
};

// With `mark`, every combo at or before the boundary is also ORed into
// R.words, and `marked` says so (not when the target exceeds the total or the
// bin overflows): the bins before the selected one from a ballot in pass 2,
// the selected bin's combos from the candidates once the boundary is known.
template <int WK, typename Eval>
__device__ BoundK wselect_interp(Eval evs, const int32_t* __restrict__ ksz, int C,
                                 unsigned long long target, double mx, double mn, SubRow& R, bool mark,
                                 bool& marked) {
  const int t = threadIdx.x, lane = t & 63;
  marked = false;
  const double span = mx - mn;
  const double inv = span > 1e-280 ? 2048.0 / span : 0.0;
  auto bin_of = [&](double l) -> int {
    const int b = int((mx - l) * inv);
    return b < 0 ? 0 : (b < 2047 ? b : 2047);
  };
  for (int b = t; b < 2048; b += SUB_T) {
    R.hw[b] = 0ull;
    R.hk[b] = 0ull;
  }
  if (t == 0) R.ncand = 0;
  __syncthreads();
  for_combos(ksz, C, [&](int g, int sz) {
    double l;
    unsigned long long k, mass, keys;
    if (!evs(g, sz, l, k, mass, keys)) {
      R.bin[g] = 0xffff;
      return;
    }
    const int b = bin_of(l);
    R.bin[g] = uint16_t(b);
    atomicAdd(&R.hw[b], WK == 0 ? mass : keys);
    if (WK == 0) atomicAdd(&R.hk[b], keys);
  });
  __syncthreads();
  const unsigned long long w0 = R.hw[2 * t], w1 = R.hw[2 * t + 1];
  const unsigned long long k0 = WK == 0 ? R.hk[2 * t] : w0, k1 = WK == 0 ? R.hk[2 * t + 1] : w1;
  unsigned long long tw, tk;
  const unsigned long long pw = bscan<unsigned long long>(w0 + w1, R.wsum, tw);
  const unsigned long long pk = bscan<unsigned long long>(k0 + k1, R.wsum, tk);
  if (t == 0) R.sel_bin = -1;
  __syncthreads();
  const unsigned long long rem0 = target;
  if (pw < rem0 && rem0 <= pw + w0) {
    R.sel_bin = 2 * t;
    R.sel_w = pw;
    R.sel_k = pk;
  } else if (pw + w0 < rem0 && rem0 <= pw + w0 + w1) {
    R.sel_bin = 2 * t + 1;
    R.sel_w = pw + w0;
    R.sel_k = pk + k0;
  }
  __syncthreads();
  const int sb = R.sel_bin;
  if (sb < 0) return BoundK{Boundary{0ull, C}, (long long)tk, true};  // target beyond the total
  const unsigned long long rem = rem0 - R.sel_w;
  const unsigned long long kbefore = R.sel_k;
  // Only the selected bin's combos are evaluated again.  A wave's lanes take
  // 64 consecutive combos: two whole mask words.
  for (int g0 = t - lane; g0 < C; g0 += SUB_T) {
    const int g = g0 + lane;
    const int b = g < C ? int(R.bin[g]) : 0xffff;
    if (mark) {
      const unsigned long long bits = __ballot(b < sb);
      if (lane == 0) R.words[g0 >> 5] |= uint32_t(bits);
      if (lane == 32 && g < C) R.words[(g0 >> 5) + 1] |= uint32_t(bits >> 32);
    }
    if (b != sb) continue;
    double l;
    unsigned long long k, mass, keys;
    evs(g, ksz[g], l, k, mass, keys);
    const int slot = atomicAdd(&R.ncand, 1);
    if (slot < CAND) {
      R.ck[slot] = k;
      R.cg[slot] = g;
      R.cw[slot] = WK == 0 ? mass : keys;
      R.ckeys[slot] = uint32_t(keys);
    }
  }
  if (t == 0) R.tie_g = -1;
  __syncthreads();
  const int m = R.ncand;
  if (m > CAND) return BoundK{Boundary{0ull, -1}, 0, false};
  if (t < m) {
    const unsigned long long mk = R.ck[t];
    const int mg = R.cg[t];
    unsigned long long sw = 0, sk = 0;
    for (int j = 0; j < m; ++j) {
      const unsigned long long kj = R.ck[j];
      if (kj < mk || (kj == mk && R.cg[j] < mg)) {
        sw += R.cw[j];
        sk += R.ckeys[j];
      }
    }
    const unsigned long long wt = R.cw[t];
    if (sw < rem && rem <= sw + wt) {
      R.tie_g = mg;
      R.tie_key = mk;
      R.tie_keys = (long long)(kbefore + sk + R.ckeys[t]);
    }
  }
  __syncthreads();
  // the bin's weight reaches rem, so exactly one candidate matched
  const BoundK r{Boundary{R.tie_key, R.tie_g}, R.tie_keys, true};
  if (mark) {
    if (t < m && before_or_at(R.ck[t], R.cg[t], r.b)) atomicOr(&R.words[R.cg[t] >> 5], 1u << (R.cg[t] & 31));
    marked = true;
  }
  __syncthreads();
  return r;
}

// c ? x : y, field by field: a select between two whole structs becomes a
// select between their addresses, which puts both in private memory.
__device__ __forceinline__ BoundK pick_bound(bool c, const BoundK& x, const BoundK& y) {
  return BoundK{Boundary{c ? x.b.key : y.b.key, c ? x.b.g : y.b.g}, c ? x.keys : y.keys,
                c ? x.ok : y.ok};
}

__device__ __forceinline__ bool later(const Boundary& a, const Boundary& b, int C) {
  // is boundary a later in rank order than b (C = past every combo)?
  if (a.g == C) return b.g != C;
  if (b.g == C) return false;
  return a.key > b.key || (a.key == b.key && a.g > b.g);
}

// keys per combo, from the offsets
__global__ void sizes_kernel(const int32_t* __restrict__ k_off, int C, int32_t* __restrict__ ksz) {
  const int h = blockIdx.y;
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= C) return;
  ksz[size_t(h) * C + g] = k_off[size_t(h) * (C + 1) + g + 1] - k_off[size_t(h) * (C + 1) + g];
}

// The online mode runs twice: pass 0 finds every row's initial boundary and
// adds its keys to the head's total, keeping the row's logit range and
// boundary in `state` (5 words per row); pass 1 starts from that state.
__global__ __launch_bounds__(SUB_T) void select_subspace(SelectArgs a, const int32_t* __restrict__ kszs,
                                                         unsigned long long* __restrict__ acc,
                                                         long long* __restrict__ state, int pass) {
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
  // lookup tables: T[slice][cluster] one wave-wide dot at a time (lanes over
  // the slice's columns, then a butterfly sum; lane 0's result is kept)
  for (int pr = w; pr < 3 * Cs; pr += SUB_T / 64) {
    const int sl = pr / Cs, c = pr - sl * Cs;
    // (constant indices only: a runtime index into the argument struct would
    // copy it to private memory in every thread)
    const int off = sl == 0 ? 0 : (sl == 1 ? a.dims[0] : a.dims[0] + a.dims[1]);
    const int dsl = sl == 0 ? a.dims[0] : (sl == 1 ? a.dims[1] : a.dims[2]);
    const float* qb = a.qbar + row * d + off;
    const float* cb = a.kbar + (size_t(h) * 3 * Cs + pr) * d + off;
    double sdot = 0.0;
    for (int col = lane; col < dsl; col += 64) sdot = fma(double(qb[col]), double(cb[col]), sdot);
    for (int o = 32; o > 0; o >>= 1) sdot += __shfl_xor(sdot, o, 64);
    if (lane == 0) R.T[sl][c] = sdot * a.scale;
  }
  for (int z = t; z < LOGT; z += SUB_T) R.lt[z] = z > 0 ? log(double(z)) : -__builtin_huge_val();
  for (int x = t; x < W; x += SUB_T) R.words[x] = 0u;
  __syncthreads();
  const int32_t* ksz = kszs + size_t(h) * C;  // keys per combo
  const int Cs2 = Cs * Cs;
  // g / Cs and g / Cs^2 as a multiply by ceil(2^31 / divisor) and a shift:
  // exact for every g < 2^15 and divisor <= 1024 (combos < 32^3)
  const uint32_t m1 = uint32_t(((1ull << 31) + Cs - 1) / Cs);
  const uint32_t m2 = uint32_t(((1ull << 31) + Cs2 - 1) / Cs2);
  // logit of combo g given its size sz; false for an empty combo
  // (a power-of-two Cs, the usual case, takes shifts and masks instead)
  const int csh = (Cs & (Cs - 1)) == 0 ? __builtin_ctz(Cs) : -1;
  auto logit_sz = [&](int g, int sz, double& l) -> bool {
    if (sz <= 0) return false;
    int c0, c1, c2;
    if (csh >= 0) {
      c0 = g >> (2 * csh);
      c1 = (g >> csh) & (Cs - 1);
      c2 = g & (Cs - 1);
    } else {
      const int q1 = int((uint64_t(uint32_t(g)) * m1) >> 31);
      c0 = int((uint64_t(uint32_t(g)) * m2) >> 31);
      c1 = q1 - c0 * Cs;
      c2 = g - q1 * Cs;
    }
    l = (R.T[0][c0] + R.T[1][c1]) + R.T[2][c2];
    // (the rare large combo takes ln directly: a select between the LDS table
    // and a global one would become one flat load waiting on every counter)
    if (a.weighted) l += sz < LOGT ? R.lt[sz] : log(double(sz));
    return true;
  };
  auto logit = [&](int g, double& l, int& sz) -> bool {
    sz = ksz[g];
    return logit_sz(g, sz, l);
  };
  const bool resume = online && pass == 1;
  long long* rs = state + row * 5;
  const double P = a.top_p;
  // no mass target (or none left to find): no normaliser, and the logit range
  // only places the interpolation bins, so bounds serve
  const bool need_mass = P > 0.0 && P < 1.0 && !resume;
  // max logit, normaliser, order-key range
  double mx = -__builtin_huge_val(), mn = __builtin_huge_val();
  if (resume) {
    mx = __longlong_as_double(rs[0]);
    mn = __longlong_as_double(rs[1]);
  } else if (need_mass) {
    for_combos(ksz, C, [&](int g, int sz) {
      double l;
      if (logit_sz(g, sz, l)) {
        mx = fmax(mx, l);
        mn = fmin(mn, l);
      }
    });
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
  } else {
    // Bounds on every logit: the sums of the slices' extremes, added in the
    // logits' own order (rounding is monotone), with ln(size) in [0, ln N]
    // given a margin far above the error of ln.  Each half-wave reduces
    // clusters lane & 31 < Cs.
    const int c = lane & 31;
    double hi[3], lo[3];
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
      hi[sl] = c < Cs ? R.T[sl][c] : -__builtin_huge_val();
      lo[sl] = c < Cs ? R.T[sl][c] : __builtin_huge_val();
      for (int o = 16; o > 0; o >>= 1) {
        hi[sl] = fmax(hi[sl], __shfl_xor(hi[sl], o, 64));
        lo[sl] = fmin(lo[sl], __shfl_xor(lo[sl], o, 64));
      }
    }
    mx = (hi[0] + hi[1]) + hi[2];
    mn = (lo[0] + lo[1]) + lo[2];
    if (a.weighted) {
      mx += log(double(a.N)) + 1e-9;
      mn -= 1e-9;
    }
  }
  double Z = 1.0;
  if (need_mass) {
    double zs = 0.0;
    for_combos(ksz, C, [&](int g, int sz) {
      double l;
      if (logit_sz(g, sz, l)) zs += exp(l - mx);
    });
    for (int o = 32; o > 0; o >>= 1) zs += __shfl_xor(zs, o, 64);
    if (lane == 0) R.dred[w] = zs;
    __syncthreads();
    Z = 0.0;
    for (int j = 0; j < SUB_T / 64; ++j) Z += R.dred[j];
    __syncthreads();
  }
  const unsigned long long kmin = order_key(mx), kmax = order_key(mn);
  auto evs = [&](int g, int sz, double& l, unsigned long long& k, unsigned long long& mass,
                 unsigned long long& keys) -> bool {
    if (!logit_sz(g, sz, l)) return false;
    k = order_key(l);
    mass = (unsigned long long)llrint(exp(l - mx) / Z * MASS_ONE);
    keys = (unsigned long long)sz;
    return true;
  };
  auto ev = [&](int g, unsigned long long& k, unsigned long long& mass, unsigned long long& keys) -> bool {
    double l;
    return evs(g, ksz[g], l, k, mass, keys);
  };
  const int Cfull = C;
  const Boundary b0{0ull, -1};  // before every combo
  auto keys_through = [&](const Boundary& b) -> long long {
    // keys of every combo up to and including the boundary: the predicate
    // the mask is built from, so counts and mask agree by construction
    if (b.g < 0) return 0;
    unsigned long long sk = 0;
    for (int g = t; g < C; g += SUB_T) {
      double l;
      int sz;
      if (!logit(g, l, sz)) continue;
      if (b.g == Cfull || before_or_at(order_key(l), g, b)) sk += (unsigned long long)sz;
    }
    unsigned long long tot;
    bscan<unsigned long long>(sk, R.wsum, tot);
    return (long long)tot;
  };
  // boundary of a cumulative target and the keys through it
  // Without the online pass the row's mask is the union of what the
  // selections mark (each marks a prefix in rank order; the mask is the
  // longest); when one of them cannot, a last pass builds it instead.
  const bool mark = !online;
  bool words_ok = mark;
  auto select_mass = [&](unsigned long long target) -> BoundK {
    bool marked;
    BoundK r = wselect_interp<0>(evs, ksz, C, target, mx, mn, R, mark, marked);
    words_ok &= marked;
    if (!r.ok) {
      r.b = wselect<0>(ev, C, target, kmin, kmax, R);
      r.keys = keys_through(r.b);
    }
    return r;
  };
  auto select_keys = [&](unsigned long long target) -> BoundK {
    bool marked;
    BoundK r = wselect_interp<1>(evs, ksz, C, target, mx, mn, R, mark, marked);
    words_ok &= marked;
    if (!r.ok) {
      r.b = wselect<1>(ev, C, target, kmin, kmax, R);
      r.keys = keys_through(r.b);
    }
    return r;
  };
  BoundK binit{b0, 0, true};
  if (resume) {
    binit = BoundK{Boundary{(unsigned long long)rs[2], int(rs[3])}, rs[4], true};
  } else {
    BoundK bp{b0, 0, true}, bf{b0, 0, true};
    if (P >= 1.0) {
      bp = BoundK{Boundary{0ull, Cfull}, keys_through(Boundary{0ull, Cfull}), true};
      words_ok = false;
    } else if (P > 0.0) {
      bp = select_mass((unsigned long long)llrint(P * MASS_ONE));
    }
    // Keys grow along rank order, so when the Top-p boundary already holds
    // the floor's keys the floor's boundary is at or before it.
    if (a.floor_units > 0 && (bp.b.g < 0 || bp.keys < a.floor_units))
      bf = select_keys((unsigned long long)a.floor_units);
    binit = pick_bound(bp.b.g < 0 || (bf.b.g >= 0 && later(bf.b, bp.b, Cfull)), bf, bp);
  }
  const long long n_init = binit.keys;
  if (online && pass == 0) {
    if (t == 0) {
      atomicAdd(&acc[h], (unsigned long long)((long long)qsize * n_init));
      if (a.init_counts) a.init_counts[row] = int(n_init);
      rs[0] = __double_as_longlong(mx);
      rs[1] = __double_as_longlong(mn);
      rs[2] = (long long)binit.b.key;
      rs[3] = binit.b.g;
      rs[4] = n_init;
    }
    return;
  }
  BoundK bfin_k = binit;
  int kh = 0;
  if (online) {
    const long long A = (long long)acc[h];
    kh = int((A + a.N - 1) / a.N);
    if (n_init < kh) {
      const BoundK bk = select_keys((unsigned long long)kh);
      bfin_k = pick_bound(binit.b.g < 0 || later(bk.b, binit.b, Cfull), bk, binit);
    }
  }
  const Boundary bfin = bfin_k.b;
  const long long n_fin = bfin_k.keys;
  if (words_ok) {
    for (int x = t; x < W; x += SUB_T) a.mask[row * W + x] = R.words[x];
  }
  // A wave's 64 lanes hold 64 consecutive combos (two whole mask words) at
  // every step, so the words are written from a ballot.
  if (!words_ok) {
    for_combo_waves(ksz, C, [&](int g0, int sz) {
      const int g = g0 + lane;
      double l;
      unsigned long long k = 0, m2, ky;
      const bool in = bfin.g >= 0 && sz > 0 && evs(g, sz, l, k, m2, ky) &&
                      (bfin.g == Cfull || before_or_at(k, g, bfin));
      const unsigned long long bits = __ballot(in);
      if (lane == 0) a.mask[row * W + (g0 >> 5)] = uint32_t(bits);
      if (lane == 32 && g < C) a.mask[row * W + (g0 >> 5) + 1] = uint32_t(bits >> 32);
    });
  }
  if (t == 0) {
    a.counts[row] = int(n_fin);
    if (a.init_counts) a.init_counts[row] = int(n_init);
    if (i == 0) a.head_topk[h] = kh;
  }
}


// --------------------------------------------------------------------------
// key clusters
// --------------------------------------------------------------------------
// Logits of a head: LT x LT output tiles, (LT/16) x (LT/16) outputs per
// thread (rows ti + 16 r, columns tj + 16 c), so each LDS read feeds LT/16
// FMAs; each output sums over d in order, one fp64 FMA per column.  64-wide
// tiles halve the LDS reads per FMA; 32-wide ones keep small problems spread
// over more workgroups.
constexpr int LC = 32;   // columns of d staged at a time
template <int LT>
__global__ __launch_bounds__(256) void logits_kernel(SelectArgs a, double* __restrict__ L) {
  constexpr int RB = LT / 16;  // outputs per thread along each axis
  __shared__ double qs[LT][LC + 1], ks[LT][LC + 1];
  const int h = blockIdx.z, i0 = blockIdx.y * LT, j0 = blockIdx.x * LT, t = threadIdx.x;
  const int ti = t >> 4, tj = t & 15;
  double acc[RB][RB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[r][c] = 0.0;
  for (int c0 = 0; c0 < a.d; c0 += LC) {
    for (int e = t; e < LT * LC; e += 256) {
      const int r = e / LC, c = e % LC;
      const int qi = i0 + r, kj = j0 + r;
      qs[r][c] = qi < a.Cq ? double(a.qbar[(size_t(h) * a.Cq + qi) * a.d + c0 + c]) : 0.0;
      ks[r][c] = kj < a.Ck ? double(a.kbar[(size_t(h) * a.Ck + kj) * a.d + c0 + c]) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < LC; ++c) {
      double qv[RB], kv[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) qv[r] = qs[ti + 16 * r][c];
#pragma unroll
      for (int cc = 0; cc < RB; ++cc) kv[cc] = ks[tj + 16 * cc][c];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int cc = 0; cc < RB; ++cc) acc[r][cc] = fma(qv[r], kv[cc], acc[r][cc]);
    }
    __syncthreads();
  }
  const int32_t* ko = a.k_off + size_t(h) * (a.Ck + 1);
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int cc = 0; cc < RB; ++cc) {
      const int i = i0 + ti + 16 * r, j = j0 + tj + 16 * cc;
      if (i >= a.Cq || j >= a.Ck) continue;
      const int sz = ko[j + 1] - ko[j];
      double l = -__builtin_huge_val();
      if (sz > 0) {
        l = acc[r][cc] * a.scale;
        if (a.weighted) l += log(double(sz));
      }
      L[(size_t(h) * a.Cq + i) * a.Ck + j] = l;
    }
}

constexpr int SW_M = SEL_MAX / 64;  // entries per lane
constexpr unsigned long long NO_KEY = ~0ull;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename V>
__device__ __forceinline__ V wave_incl_scan(V v) {
  const int lane = __lane_id();
  for (int o = 1; o < 64; o <<= 1) {
    const V y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// (key, j) position in rank order; j = INT_MAX: past every entry
struct WBound {
  unsigned long long key;
  int j;
};

// One wavefront: entry j = lane + 64 m (m < SW_M) has order key key[m]
// (NO_KEY: absent) and weight wt[m].  Returns the first entry, in ascending
// (key, j), at which the cumulative weight reaches target (>= 1), or
// {NO_KEY, INT_MAX} when the total stays below it.  8-bit radix passes over
// the bits below the common prefix of the keys, then the equal keys in j order.
__device__ WBound wave_select(const unsigned long long (&key)[SW_M], const unsigned long long (&wt)[SW_M],
                              unsigned long long target, unsigned long long* hist) {
  const int lane = __lane_id();
  unsigned long long mn = NO_KEY, mx = 0ull;
#pragma unroll
  for (int m = 0; m < SW_M; ++m)
    if (key[m] != NO_KEY) {
      mn = key[m] < mn ? key[m] : mn;
      mx = key[m] > mx ? key[m] : mx;
    }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long a = __shfl_xor(mn, o, 64), b = __shfl_xor(mx, o, 64);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  const WBound all{NO_KEY, 0x7fffffff};
  if (mn == NO_KEY) return all;
  unsigned long long prefix = mn, rem = target;
  int hb = mn == mx ? -1 : 63 - __clzll(mn ^ mx);
  if (hb >= 0) prefix = hb == 63 ? 0ull : (mn & ~((2ull << hb) - 1ull));
  while (hb >= 0) {
    const int shift = max(hb - 7, 0);
    const unsigned long long dmask = (1ull << (hb - shift + 1)) - 1ull;
    const int above = hb + 1;
    for (int b = lane; b < 256; b += 64) hist[b] = 0ull;
    wave_sync();
#pragma unroll
    for (int m = 0; m < SW_M; ++m)
      if (key[m] != NO_KEY && (above >= 64 || (key[m] >> above) == (prefix >> above)))
        atomicAdd(&hist[int((key[m] >> shift) & dmask)], wt[m]);
    wave_sync();
    unsigned long long c[4], loc = 0ull;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = hist[4 * lane + q];
      loc += c[q];
    }
    const unsigned long long incl = wave_incl_scan(loc);
    unsigned long long run = incl - loc;
    int bin = -1;
    unsigned long long below = 0ull;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (bin < 0 && run < rem && rem <= run + c[q]) {
        bin = 4 * lane + q;
        below = run;
      }
      run += c[q];
    }
    const uint64_t bal = __ballot(bin >= 0);
    wave_sync();
    if (!bal) return all;
    const int lead = __ffsll((unsigned long long)bal) - 1;
    bin = __shfl(bin, lead, 64);
    below = __shfl(below, lead, 64);
    prefix |= (unsigned long long)bin << shift;
    rem -= below;
    if (shift == 0) break;
    hb = shift - 1;
  }
  unsigned long long run = 0ull;
#pragma unroll
  for (int m = 0; m < SW_M; ++m) {
    const bool f = key[m] == prefix;
    const unsigned long long w = f ? wt[m] : 0ull;
    const unsigned long long incl = wave_incl_scan(w);
    const unsigned long long tot = __shfl(incl, 63, 64);
    const uint64_t bal = __ballot(f && run + incl - w < rem && rem <= run + incl);
    if (bal) return WBound{prefix, __ffsll((unsigned long long)bal) - 1 + 64 * m};
    run += tot;
  }
  return all;
}

__device__ __forceinline__ bool through(unsigned long long k, int j, const WBound& b) {
  return k != NO_KEY && (b.j == 0x7fffffff || k < b.key || (k == b.key && j <= b.j));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wavefront per query cluster (four per workgroup).
__global__ __launch_bounds__(256) void select_wave(SelectArgs a, const double* __restrict__ L,
                                                   unsigned long long* __restrict__ acc,
                                                   const int32_t* __restrict__ pool_cnt, int pass) {
  __shared__ unsigned long long hist[4][256];
  __shared__ uint32_t words[4][SEL_MAX / 32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wv, h = blockIdx.y;
  if (i >= a.Cq) return;
  const int Ck = a.Ck, W = ceil_div(Ck, 32);
  const size_t row = size_t(h) * a.Cq + i;
  const int32_t* qo = a.q_off + size_t(h) * (a.Cq + 1);
  const int qsize = qo[i + 1] - qo[i];
  const bool online = a.online != 0;
  if (qsize == 0) {  // selects nothing and adds nothing to A_h
    if (!online || pass == 1) {
      for (int x = lane; x < W; x += 64) a.mask[row * W + x] = 0u;
      if (lane == 0) {
        a.counts[row] = 0;
        if (a.init_counts) a.init_counts[row] = 0;
        if (i == 0) a.head_topk[h] = online ? int(((long long)acc[h] + a.N - 1) / a.N) : 0;
      }
    } else if (lane == 0 && a.init_counts) {
      a.init_counts[row] = 0;
    }
    return;
  }
  const double* lr = L + row * Ck;
  double l[SW_M];
  double mx = -__builtin_huge_val();
#pragma unroll
  for (int m = 0; m < SW_M; ++m) {
    const int j = lane + 64 * m;
    l[m] = j < Ck ? lr[j] : -__builtin_huge_val();
    mx = fmax(mx, l[m]);
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  const double P = a.top_p;
  const bool pooled = pool_cnt && pool_cnt[row] >= 0;
  // probabilities only where the rule reads them: a mass target strictly
  // between 0 and 1, or the statistical threshold (a fixed floor needs the
  // ranking alone)
  const bool need_mass = !pooled && a.rule != SA_RULE_STAT && P > 0.0 && P < 1.0;
  const bool need_z = !pooled && (need_mass || a.rule == SA_RULE_STAT);
  double z = 0.0;
  if (need_z) {
#pragma unroll
    for (int m = 0; m < SW_M; ++m)
      if (l[m] != -__builtin_huge_val()) z += exp(l[m] - mx);
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
  }
  unsigned long long key[SW_M], ms[SW_M], one[SW_M];
  int nv = 0;
#pragma unroll
  for (int m = 0; m < SW_M; ++m) {
    const bool v = l[m] != -__builtin_huge_val();
    key[m] = v ? order_key(l[m]) : NO_KEY;
    ms[m] = 0ull;
    if (need_mass && v) ms[m] = (unsigned long long)llrint(exp(l[m] - mx) / z * MASS_ONE);
    one[m] = v ? 1ull : 0ull;
    nv += v ? 1 : 0;
  }
  const int Vn = wave_sum_i32(nv);
  auto count_through = [&](const WBound& b) {
    int c = 0;
#pragma unroll
    for (int m = 0; m < SW_M; ++m) c += through(key[m], lane + 64 * m, b) ? 1 : 0;
    return wave_sum_i32(c);
  };
  int np;
  if (pooled) np = pool_cnt[row];  // decided by the row's pool
  else if (a.rule == SA_RULE_STAT) {
    // BSA statistical threshold: mean + lambda * population std of the row's
    // probabilities (fixed-order sums), then the units at or above it
    double pr[SW_M], s1 = 0.0;
#pragma unroll
    for (int m = 0; m < SW_M; ++m) {
      pr[m] = key[m] != NO_KEY ? exp(l[m] - mx) / z : 0.0;
      s1 += pr[m];
    }
    for (int o = 32; o > 0; o >>= 1) s1 += __shfl_xor(s1, o, 64);
    const double mu = s1 / double(Vn);
    double s2 = 0.0;
#pragma unroll
    for (int m = 0; m < SW_M; ++m)
      if (key[m] != NO_KEY) s2 += (pr[m] - mu) * (pr[m] - mu);
    for (int o = 32; o > 0; o >>= 1) s2 += __shfl_xor(s2, o, 64);
    const double th = mu + a.stat_lambda * sqrt(s2 / double(Vn));
    int c = 0;
#pragma unroll
    for (int m = 0; m < SW_M; ++m) c += (key[m] != NO_KEY && pr[m] >= th) ? 1 : 0;
    np = wave_sum_i32(c);
  } else if (P >= 1.0) np = Vn;
  else if (P <= 0.0) np = 0;
  else np = count_through(wave_select(key, ms, (unsigned long long)llrint(P * MASS_ONE), hist[wv]));
  const int nf = a.floor_units > 0 ? min(a.floor_units, Vn) : 0;
  const int t_init = max(np, nf);
  if (online && pass == 0) {
    if (lane == 0) {
      atomicAdd(&acc[h], (unsigned long long)((long long)qsize * t_init));
      if (a.init_counts) a.init_counts[row] = t_init;
    }
    return;
  }
  int t_fin = t_init, kh = 0;
  if (online) {
    kh = int(((long long)acc[h] + a.N - 1) / a.N);
    if (t_init < kh) t_fin = min(kh, Vn);
  }
  uint32_t* wd = words[wv];
  for (int x = lane; x < W; x += 64) wd[x] = 0u;
  wave_sync();
  if (t_fin > 0) {
    const WBound b = wave_select(key, one, (unsigned long long)t_fin, hist[wv]);
#pragma unroll
    for (int m = 0; m < SW_M; ++m) {
      const int j = lane + 64 * m;
      if (through(key[m], j, b)) atomicOr(&wd[j >> 5], 1u << (j & 31));
    }
  }
  wave_sync();
  for (int x = lane; x < W; x += 64) a.mask[row * W + x] = wd[x];
  if (lane == 0) {
    a.counts[row] = t_fin;
    if (a.init_counts) a.init_counts[row] = t_init;
    if (i == 0) a.head_topk[h] = kh;
  }
}

// --------------------------------------------------------------------------
// Competition domains (EG-Sparse: low-entropy heads share a grouped
// cross-head pool, high-entropy heads keep per-row selection; VMoBA: global
// block selection over a whole head).  A pool's (head, row, unit) pairs
// compete by proxy probability p_ij (descending; ties by head, row, unit),
// each carrying the mass |Q_i| p_ij / N in 2^-52 fixed point; the pool keeps
// the shortest prefix whose mass reaches top_p times its number of heads.
// The pooled pairs of a row are the first of its own ranking, so the pool
// hands each row a Top-p count and the per-row selection does the rest
// (floor, online Top-k, mask).
// --------------------------------------------------------------------------
constexpr int PBIN = 2048;  // radix bins (11-bit digits of the 64-bit keys)

struct PoolState {
  unsigned long long prefix;  // key digits fixed so far
  long long rem;              // mass still needed inside the keys of that prefix
  int all;                    // the pool's whole mass stays below the target: take every pair
  int heads;                  // heads in the pool
};

// pool of head h: -1 = per-row selection
__device__ __forceinline__ int pool_of(const SelectArgs& a, const double* E, int h) {
  if (a.domain == SA_DOMAIN_HEAD) return h;
  if (a.domain == SA_DOMAIN_GROUP && E[h] < a.max_entropy) return h / a.group;
  return -1;
}
__host__ __device__ inline int pool_slots(int domain, int group) { return domain == SA_DOMAIN_GROUP ? group : 1; }

// One wavefront per row: max, normaliser and normalised entropy of the row's
// proxy distribution (sums in a fixed order: lane partials in unit order, then
// a fixed butterfly).
__global__ __launch_bounds__(256) void rowstat_kernel(SelectArgs a, const double* __restrict__ L,
                                                      double* __restrict__ stat) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)a.H * a.Cq) return;
  const double* lr = L + row * a.Ck;
  double mx = -__builtin_huge_val();
  int nv = 0;
  for (int j = lane; j < a.Ck; j += 64) {
    const double l = lr[j];
    if (l != -__builtin_huge_val()) {
      mx = fmax(mx, l);
      ++nv;
    }
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  nv = wave_sum_i32(nv);
  double z = 0.0;
  for (int j = lane; j < a.Ck; j += 64) {
    const double l = lr[j];
    if (l != -__builtin_huge_val()) z += exp(l - mx);
  }
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
  double plp = 0.0;
  for (int j = lane; j < a.Ck; j += 64) {
    const double l = lr[j];
    if (l != -__builtin_huge_val()) {
      const double pr = exp(l - mx) / z;
      if (pr > 0.0) plp += pr * log(pr);
    }
  }
  for (int o = 32; o > 0; o >>= 1) plp += __shfl_xor(plp, o, 64);
  if (lane == 0) {
    stat[3 * row] = mx;
    stat[3 * row + 1] = z;
    stat[3 * row + 2] = nv > 1 ? -plp / log(double(nv)) : 0.0;
  }
}

// One workgroup per head: E_h = sum_i |Q_i| ent_i / N in a fixed order.
__global__ __launch_bounds__(256) void head_entropy_kernel(SelectArgs a, const double* __restrict__ stat,
                                                           double* __restrict__ E) {
  __shared__ double part[256];
  const int h = blockIdx.x, t = threadIdx.x;
  const int32_t* qo = a.q_off + size_t(h) * (a.Cq + 1);
  double acc = 0.0;
  for (int i = t; i < a.Cq; i += 256)
    acc += double(qo[i + 1] - qo[i]) * stat[3 * (size_t(h) * a.Cq + i) + 2];
  part[t] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) part[t] += part[t + o];
    __syncthreads();
  }
  if (t == 0) {
    const double e = part[0] / double(a.N);
    E[h] = e;
    if (a.head_entropy) a.head_entropy[h] = e;
  }
}

__global__ void fill_i32_kernel(int32_t* p, long long n, int v) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// probability, order key and fixed-point mass of pair (row, j)
struct PairVal {
  unsigned long long key, w;
  bool valid;
};
__device__ __forceinline__ PairVal pair_val(const double* lr, const double* st, int j, double qscale) {
  const double l = lr[j];
  PairVal v{0ull, 0ull, false};
  if (l == -__builtin_huge_val()) return v;
  const double pr = exp(l - st[0]) / st[1];
  v.key = order_key(pr);
  v.w = (unsigned long long)llrint(pr * qscale);
  v.valid = true;
  return v;
}

// Radix pass: mass histogram of the digit below the fixed prefix, over the
// pairs of the pooled rows.  Workgroup: 16 rows (4 per wavefront) of one head
// slot of one pool.  grid (ceil(Cq/16), slots, pools).
__global__ __launch_bounds__(256) void pool_hist_kernel(SelectArgs a, const double* __restrict__ L,
                                                        const double* __restrict__ stat,
                                                        const double* __restrict__ E,
                                                        const PoolState* __restrict__ ps,
                                                        unsigned long long* __restrict__ ghist, int shift,
                                                        int width) {
  __shared__ unsigned long long hist[PBIN];
  const int g = blockIdx.z, slot = blockIdx.y, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int h = a.domain == SA_DOMAIN_GROUP ? g * a.group + slot : g;
  if (h >= a.H || pool_of(a, E, h) != g || ps[g].all) return;
  for (int b = t; b < PBIN; b += 256) hist[b] = 0ull;
  __syncthreads();
  const int above = shift + width;
  const unsigned long long pre = ps[g].prefix;
  const unsigned long long dmask = (1ull << width) - 1ull;
  const int32_t* qo = a.q_off + size_t(h) * (a.Cq + 1);
  for (int r = 0; r < 4; ++r) {
    const int i = blockIdx.x * 16 + wv * 4 + r;
    if (i >= a.Cq) break;
    const int qs = qo[i + 1] - qo[i];
    if (qs == 0) continue;
    const size_t row = size_t(h) * a.Cq + i;
    const double qscale = double(qs) / double(a.N) * MASS_ONE;
    for (int j = lane; j < a.Ck; j += 64) {
      const PairVal v = pair_val(L + row * a.Ck, stat + 3 * row, j, qscale);
      if (!v.valid || v.w == 0ull) continue;
      if (above < 64 && (v.key >> above) != (pre >> above)) continue;
      atomicAdd(&hist[(v.key >> shift) & dmask], v.w);
    }
  }
  __syncthreads();
  unsigned long long* gh = ghist + size_t(g) * PBIN;
  for (int b = t; b < PBIN; b += 256)
    if (hist[b]) atomicAdd(&gh[b], hist[b]);
}

// One thread per pool: its heads and its target, top_p times their number.
__global__ void pool_init_kernel(SelectArgs a, const double* __restrict__ E, PoolState* __restrict__ ps,
                                 int pools) {
  const int g = blockIdx.x * 64 + threadIdx.x;
  if (g >= pools) return;
  int m = 0;
  for (int s = 0; s < pool_slots(a.domain, a.group); ++s) {
    const int h = a.domain == SA_DOMAIN_GROUP ? g * a.group + s : g;
    if (h < a.H && pool_of(a, E, h) == g) ++m;
  }
  ps[g].heads = m;
  ps[g].prefix = 0ull;
  ps[g].rem = llrint(a.top_p * double(m) * MASS_ONE);
  ps[g].all = 0;
}

// One workgroup per pool: the bin where the cumulative mass reaches the
// remaining target; fixes that digit.  Clears the histogram for the next pass.
__global__ __launch_bounds__(256) void pool_pick_kernel(PoolState* __restrict__ ps,
                                                        unsigned long long* __restrict__ ghist, int shift) {
  __shared__ unsigned long long wsum[16];
  __shared__ int sel_bin;
  __shared__ unsigned long long sel_pre;
  const int g = blockIdx.x, t = threadIdx.x;
  unsigned long long* gh = ghist + size_t(g) * PBIN;
  if (t == 0) sel_bin = -1;
  __syncthreads();
  if (ps[g].heads == 0 || ps[g].all) {
    for (int b = t; b < PBIN; b += 256) gh[b] = 0ull;
    return;
  }
  constexpr int BPT = PBIN / 256;
  unsigned long long c[BPT], loc = 0ull;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = gh[t * BPT + q];
    loc += c[q];
  }
  unsigned long long tot;
  unsigned long long pre = bscan<unsigned long long>(loc, wsum, tot);
  const unsigned long long rem = (unsigned long long)ps[g].rem;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    if (pre < rem && rem <= pre + c[q]) {
      sel_bin = t * BPT + q;
      sel_pre = pre;
    }
    pre += c[q];
  }
  __syncthreads();
  for (int b = t; b < PBIN; b += 256) gh[b] = 0ull;
  if (t == 0) {
    if (sel_bin < 0) {
      ps[g].all = 1;  // the pool's mass never reaches the target: every pair
    } else {
      ps[g].prefix |= (unsigned long long)sel_bin << shift;
      ps[g].rem = (long long)(rem - sel_pre);
    }
  }
}

// Per pooled row: pairs before the boundary key (all pairs if the pool takes
// everything), plus the count and mass of its pairs on the boundary key.
__global__ __launch_bounds__(256) void pool_count_kernel(SelectArgs a, const double* __restrict__ L,
                                                         const double* __restrict__ stat,
                                                         const double* __restrict__ E,
                                                         const PoolState* __restrict__ ps,
                                                         int32_t* __restrict__ pool_cnt,
                                                         int32_t* __restrict__ tie_n,
                                                         unsigned long long* __restrict__ tie_w) {
  const int g = blockIdx.z, slot = blockIdx.y, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int h = a.domain == SA_DOMAIN_GROUP ? g * a.group + slot : g;
  if (h >= a.H || pool_of(a, E, h) != g) return;
  const unsigned long long K = ps[g].prefix;
  const bool all = ps[g].all != 0;
  const int32_t* qo = a.q_off + size_t(h) * (a.Cq + 1);
  for (int r = 0; r < 4; ++r) {
    const int i = blockIdx.x * 16 + wv * 4 + r;
    if (i >= a.Cq) break;
    const int qs = qo[i + 1] - qo[i];
    const size_t row = size_t(h) * a.Cq + i;
    const double qscale = double(qs) / double(a.N) * MASS_ONE;
    int nlt = 0, neq = 0;
    unsigned long long weq = 0ull;
    if (qs > 0) {
      for (int j = lane; j < a.Ck; j += 64) {
        const PairVal v = pair_val(L + row * a.Ck, stat + 3 * row, j, qscale);
        if (!v.valid) continue;
        if (all || v.key < K) ++nlt;
        else if (v.key == K) {
          ++neq;
          weq += v.w;
        }
      }
    }
    nlt = wave_sum_i32(nlt);
    neq = wave_sum_i32(neq);
    for (int o = 32; o > 0; o >>= 1) weq += __shfl_xor(weq, o, 64);
    if (lane == 0) {
      pool_cnt[row] = nlt;
      tie_n[row] = all ? 0 : neq;
      tie_w[row] = all ? 0ull : weq;
    }
  }
}

// One workgroup per pool: the pairs on the boundary key are taken in (head,
// row, unit) order until the remaining mass is reached.
__global__ __launch_bounds__(64) void pool_tie_kernel(SelectArgs a, const double* __restrict__ L,
                                                      const double* __restrict__ stat,
                                                      const double* __restrict__ E,
                                                      const PoolState* __restrict__ ps,
                                                      int32_t* __restrict__ pool_cnt,
                                                      const int32_t* __restrict__ tie_n,
                                                      const unsigned long long* __restrict__ tie_w) {
  const int g = blockIdx.x;
  if (threadIdx.x != 0 || ps[g].heads == 0 || ps[g].all) return;
  const unsigned long long K = ps[g].prefix;
  unsigned long long need = (unsigned long long)ps[g].rem;  // >= 1
  for (int s = 0; s < pool_slots(a.domain, a.group) && need > 0ull; ++s) {
    const int h = a.domain == SA_DOMAIN_GROUP ? g * a.group + s : g;
    if (h >= a.H || pool_of(a, E, h) != g) continue;
    const int32_t* qo = a.q_off + size_t(h) * (a.Cq + 1);
    for (int i = 0; i < a.Cq && need > 0ull; ++i) {
      const size_t row = size_t(h) * a.Cq + i;
      if (tie_n[row] == 0) continue;
      if (tie_w[row] < need) {
        pool_cnt[row] += tie_n[row];
        need -= tie_w[row];
        continue;
      }
      // the boundary row: its tied units in unit order
      const double qscale = double(qo[i + 1] - qo[i]) / double(a.N) * MASS_ONE;
      int taken = 0;
      for (int j = 0; j < a.Ck && need > 0ull; ++j) {
        const PairVal v = pair_val(L + row * a.Ck, stat + 3 * row, j, qscale);
        if (!v.valid || v.key != K) continue;
        ++taken;
        need = v.w >= need ? 0ull : need - v.w;
      }
      pool_cnt[row] += taken;
    }
  }
}

}  // namespace

size_t select_scratch(int H, int Cq, int Ck, int subspace, int domain, int group) {
  Arena a{nullptr, 0, 0};
  a.get<unsigned long long>(size_t(H));
  if (subspace) {
    a.get<int32_t>(size_t(H) * Ck);
    a.get<long long>(size_t(H) * Cq * 5);
  } else {
    a.get<double>(size_t(H) * Cq * Ck);
    if (domain != SA_DOMAIN_ROW) {
      const int pools = domain == SA_DOMAIN_GROUP ? ceil_div(H, group) : H;
      a.get<double>(size_t(H) * Cq * 3);   // row max, normaliser, entropy
      a.get<double>(size_t(H));            // head entropies
      a.get<int32_t>(size_t(H) * Cq);      // pooled Top-p counts
      a.get<int32_t>(size_t(H) * Cq);      // boundary-key pairs per row
      a.get<unsigned long long>(size_t(H) * Cq);
      a.get<PoolState>(size_t(pools));
      a.get<unsigned long long>(size_t(pools) * PBIN);
    }
  }
  return a.used;
}

hipError_t select_run(const SelectArgs& a, Arena& s, hipStream_t st) {
  unsigned long long* acc = s.get<unsigned long long>(size_t(a.H));
  dim3 g(a.Cq, a.H);
  if (a.subspace) {
    if (a.Cs > 32 || a.Ck != a.Cs * a.Cs * a.Cs) return hipErrorInvalidValue;
    int32_t* ksz = s.get<int32_t>(size_t(a.H) * a.Ck);
    long long* rstate = s.get<long long>(size_t(a.H) * a.Cq * 5);
    sizes_kernel<<<dim3(ceil_div(a.Ck, 256), a.H), 256, 0, st>>>(a.k_off, a.Ck, ksz);
    if (a.online) {
      zero_u64<<<ceil_div(a.H, 256), 256, 0, st>>>(acc, a.H);
      select_subspace<<<g, SUB_T, 0, st>>>(a, ksz, acc, rstate, 0);
      select_subspace<<<g, SUB_T, 0, st>>>(a, ksz, acc, rstate, 1);
    } else {
      select_subspace<<<g, SUB_T, 0, st>>>(a, ksz, acc, rstate, 0);
    }
    return hipGetLastError();
  }
  if (a.Ck > SEL_MAX || a.d % LC) return hipErrorInvalidValue;
  double* L = s.get<double>(size_t(a.H) * a.Cq * a.Ck);
  // 64-wide tiles when they still give about a thousand workgroups
  if (size_t(ceil_div(a.Ck, 64)) * ceil_div(a.Cq, 64) * a.H >= 1024)
    logits_kernel<64><<<dim3(ceil_div(a.Ck, 64), ceil_div(a.Cq, 64), a.H), 256, 0, st>>>(a, L);
  else
    logits_kernel<32><<<dim3(ceil_div(a.Ck, 32), ceil_div(a.Cq, 32), a.H), 256, 0, st>>>(a, L);
  int32_t* pool_cnt = nullptr;
  if (a.domain != SA_DOMAIN_ROW) {
    if (a.domain == SA_DOMAIN_GROUP && a.group < 1) return hipErrorInvalidValue;
    const int pools = a.domain == SA_DOMAIN_GROUP ? ceil_div(a.H, a.group) : a.H;
    const long long rows = (long long)a.H * a.Cq;
    double* stat = s.get<double>(size_t(rows) * 3);
    double* E = s.get<double>(size_t(a.H));
    pool_cnt = s.get<int32_t>(size_t(rows));
    int32_t* tie_n = s.get<int32_t>(size_t(rows));
    unsigned long long* tie_w = s.get<unsigned long long>(size_t(rows));
    PoolState* ps = s.get<PoolState>(size_t(pools));
    unsigned long long* ghist = s.get<unsigned long long>(size_t(pools) * PBIN);
    rowstat_kernel<<<unsigned((rows + 3) / 4), 256, 0, st>>>(a, L, stat);
    head_entropy_kernel<<<a.H, 256, 0, st>>>(a, stat, E);
    fill_i32_kernel<<<unsigned((rows + 255) / 256), 256, 0, st>>>(pool_cnt, rows, -1);
    if (a.top_p > 0.0 && a.top_p < 1.0) {
      // pooled Top-p (top_p >= 1 or <= 0 selects the same as every row alone)
      const dim3 gp(ceil_div(a.Cq, 16), pool_slots(a.domain, a.group), pools);
      fill_u64_kernel<<<unsigned((size_t(pools) * PBIN + 255) / 256), 256, 0, st>>>(ghist, size_t(pools) * PBIN);
      pool_init_kernel<<<ceil_div(pools, 64), 64, 0, st>>>(a, E, ps, pools);
      for (int hb = 63;;) {  // 11-bit digits from the top of the 64-bit keys
        const int shift = hb - 10 > 0 ? hb - 10 : 0;
        const int width = hb - shift + 1;
        pool_hist_kernel<<<gp, 256, 0, st>>>(a, L, stat, E, ps, ghist, shift, width);
        pool_pick_kernel<<<pools, 256, 0, st>>>(ps, ghist, shift);
        if (shift == 0) break;
        hb = shift - 1;
      }
      pool_count_kernel<<<gp, 256, 0, st>>>(a, L, stat, E, ps, pool_cnt, tie_n, tie_w);
      pool_tie_kernel<<<pools, 64, 0, st>>>(a, L, stat, E, ps, pool_cnt, tie_n, tie_w);
    }
  }
  const dim3 gw(ceil_div(a.Cq, 4), a.H);
  if (a.online) {
    zero_u64<<<ceil_div(a.H, 256), 256, 0, st>>>(acc, a.H);
    select_wave<<<gw, 256, 0, st>>>(a, L, acc, pool_cnt, 0);
    select_wave<<<gw, 256, 0, st>>>(a, L, acc, pool_cnt, 1);
  } else {
    select_wave<<<gw, 256, 0, st>>>(a, L, acc, pool_cnt, 0);
  }
  return hipGetLastError();
}

}  // namespace sa
