// Balanced recursive 2-means bisection into leaves of `leaf` tokens
// (ClusterAttention, English abstract: a fast recursive clustering that gives
// power-of-two cluster sizes so that block-sparse attention runs at dense
// per-pair speed).
//
// Rule of one node (n tokens, c = ceil(n/leaf) leaves needed, c >= 2): the
// left child takes leaf*ceil(c/2) tokens; the two means start at the node's
// first two tokens; each round computes
//     delta_n = ||x_n - c1||^2 - ||x_n - c2||^2 = (c2 - c1) . (2 x_n - c1 - c2)
// sends the n_left tokens first in (delta, original index) order left and
// recomputes the two means.  After `iters` rounds the node splits stably and
// the children are processed one level down (left before right, so the final
// position order is the depth-first leaf order).
//
// The tree shape depends only on (n, leaf), so every head shares one table of
// segments per level.  All heads run each level together:
//   delta  : chunked, one 16-byte slice per lane, sortable fp32 key per token
//   select : one workgroup per segment, exact k-th smallest (key, position)
//            by a radix search below the common prefix of min/max, then an
//            ordered scan over positions for ties
//   sums   : chunked fixed-order partial sums of both sides (no float atomics)
//   update : per segment, partials summed in chunk order -> the two means
//   part.  : per segment ordered scan -> stable partition of the positions

#include <vector>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int BCH = 1024;     // positions per chunk
constexpr int MAXLEV = 32;

struct LevelTabs {
  int nlev;
  int nseg[MAXLEV], nchunk[MAXLEV], sb[MAXLEV], cb[MAXLEV];
};

struct TreePlan {
  LevelTabs t;
  int total_seg, total_chunk, max_seg, max_chunk;
};

TreePlan plan_tree(int N, int L) {
  TreePlan p{};
  std::vector<int> st{0}, nn{N};
  while (true) {
    bool any = false;
    for (int n : nn)
      if (ceil_div(n, L) >= 2) any = true;
    if (!any || p.t.nlev >= MAXLEV) break;
    const int lv = p.t.nlev++;
    p.t.nseg[lv] = int(nn.size());
    p.t.sb[lv] = p.total_seg;
    p.total_seg += int(nn.size());
    int nch = 0;
    std::vector<int> st2, nn2;
    for (size_t k = 0; k < nn.size(); ++k) {
      const int c = ceil_div(nn[k], L);
      if (c >= 2) {
        const int nl = L * ceil_div(c, 2);
        nch += ceil_div(nn[k], BCH);
        st2.push_back(st[k]);
        nn2.push_back(nl);
        st2.push_back(st[k] + nl);
        nn2.push_back(nn[k] - nl);
      } else {
        st2.push_back(st[k]);
        nn2.push_back(nn[k]);
      }
    }
    p.t.nchunk[lv] = nch;
    p.t.cb[lv] = p.total_chunk;
    p.total_chunk += nch;
    p.max_seg = max(p.max_seg, p.t.nseg[lv]);
    p.max_chunk = max(p.max_chunk, nch);
    st.swap(st2);
    nn.swap(nn2);
  }
  return p;
}

// ---------------------------------------------------------------------------
// block helpers (blockDim = 1024)
// ---------------------------------------------------------------------------
template <typename V>
__device__ V block_excl_scan_1024(V v, V* wsum /*[16]*/, V& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  V x = v;
  for (int o = 1; o < 64; o <<= 1) {
    V y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  V pre = 0, tot = 0;
  for (int j = 0; j < 16; ++j) {
    if (j < w) pre += wsum[j];
    tot += wsum[j];
  }
  total = tot;
  __syncthreads();
  return pre + x - v;
}

// ---------------------------------------------------------------------------
// tree tables on the device (one workgroup of 1024 threads)
// segs: int4 {start, n, n_left (0 = leaf), first chunk (level-local)}
// chunks: int4 {segment (level-local), position, count, 0}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tree_kernel(LevelTabs tb, int N, int L, int4* segs,
                                                          int4* chunks) {
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  if (t == 0) segs[0] = make_int4(0, N, 0, 0);
  __syncthreads();
  for (int lv = 0; lv < tb.nlev; ++lv) {
    int chunk_carry = 0, child_carry = 0;
    for (int base = 0; base < tb.nseg[lv]; base += 1024) {
      const int k = base + t;
      int4 s = make_int4(0, 0, 0, 0);
      int nchunk = 0, nchild = 0, nl = 0;
      if (k < tb.nseg[lv]) {
        s = segs[tb.sb[lv] + k];
        const int c = ceil_div(s.y, L);
        if (c >= 2) {
          nl = L * ceil_div(c, 2);
          nchunk = ceil_div(s.y, BCH);
          nchild = 2;
        } else {
          nchild = 1;
        }
      }
      int tot1, tot2;
      const int cpre = block_excl_scan_1024<int>(nchunk, wsum, tot1) + chunk_carry;
      const int kpre = block_excl_scan_1024<int>(nchild, wsum, tot2) + child_carry;
      if (k < tb.nseg[lv]) {
        segs[tb.sb[lv] + k] = make_int4(s.x, s.y, nl, cpre);
        for (int c = 0; c < nchunk; ++c) {
          const int pos = s.x + c * BCH;
          chunks[tb.cb[lv] + cpre + c] = make_int4(k, pos, min(BCH, s.x + s.y - pos), 0);
        }
        if (lv + 1 < tb.nlev) {
          int4* nxt = segs + tb.sb[lv + 1] + kpre;
          if (nchild == 2) {
            nxt[0] = make_int4(s.x, nl, 0, 0);
            nxt[1] = make_int4(s.x + nl, s.y - nl, 0, 0);
          } else {
            nxt[0] = make_int4(s.x, s.y, 0, 0);
          }
        }
      }
      chunk_carry += tot1;
      child_carry += tot2;
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
  }
}

__global__ void iota_kernel(int32_t* p, int N) {
  const int h = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n < N) p[size_t(h) * N + n] = n;
}

// ---------------------------------------------------------------------------
// delta pass
// ---------------------------------------------------------------------------
template <typename T, int D>
struct RowGeo {
  static constexpr int EPV = 16 / int(sizeof(T));  // elements per 16-byte vector
  static constexpr int LPR = D / EPV;              // lanes per row
  static constexpr int RPW = 64 / LPR;             // rows per wave step
};

template <typename T, int EPV>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[EPV]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  if constexpr (sizeof(T) == 4) {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
  } else {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ x,
                                                    const int32_t* __restrict__ perm,
                                                    const int4* __restrict__ segs,
                                                    const int4* __restrict__ chunks,
                                                    const float* __restrict__ cen, int max_seg,
                                                    int N, int first, uint32_t* __restrict__ keys) {
  using G = RowGeo<T, D>;
  __shared__ float wv[D], mv[D];
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 ch = chunks[blockIdx.x];
  const int4 sg = segs[ch.x];
  const int32_t* ph = perm + size_t(h) * N;
  const T* xh = x + size_t(h) * N * D;
  if (t < D) {
    float c1, c2;
    if (first) {
      c1 = to_f(xh[size_t(ph[sg.x]) * D + t]);
      c2 = to_f(xh[size_t(ph[sg.x + 1]) * D + t]);
    } else {
      const float* c = cen + (size_t(h) * max_seg + ch.x) * 2 * D;
      c1 = c[t];
      c2 = c[D + t];
    }
    wv[t] = c2 - c1;
    mv[t] = c1 + c2;
  }
  __syncthreads();
  const int lane = t & 63, w = t >> 6;
  const int sub = lane % G::LPR, rsub = lane / G::LPR;
  float wr[G::EPV], mr[G::EPV];
#pragma unroll
  for (int e = 0; e < G::EPV; ++e) {
    wr[e] = wv[sub * G::EPV + e];
    mr[e] = mv[sub * G::EPV + e];
  }
  for (int rb = w * G::RPW; rb < ch.z; rb += 4 * G::RPW) {
    const int r = rb + rsub;
    const bool valid = r < ch.z;
    const int p = ch.y + (valid ? r : 0);
    float v[G::EPV];
    load_vec<T, G::EPV>(xh + size_t(ph[p]) * D + sub * G::EPV, v);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) acc = fmaf(wr[e], fmaf(2.f, v[e], -mr[e]), acc);
#pragma unroll
    for (int o = 1; o < G::LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
    if (valid && sub == 0) keys[size_t(h) * N + p] = sortable(acc);
  }
}

// ---------------------------------------------------------------------------
// select: exact k-th smallest (key, position) of a segment
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void select_kernel(const uint32_t* __restrict__ keys,
                                                      const int4* __restrict__ segs, int max_seg,
                                                      int N, uint2* __restrict__ thr) {
  __shared__ int hist[2048];
  __shared__ int wsum[16];
  __shared__ uint32_t red[2][16];
  __shared__ int sel_bin, sel_pos;
  const int h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int4 sg = segs[blockIdx.x];
  if (sg.z == 0) return;
  const uint32_t* u = keys + size_t(h) * N + sg.x;
  const int n = sg.y;
  int k = sg.z;  // 1-based rank of the last left element
  // min / max
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = t; i < n; i += 1024) {
    const uint32_t v = u[i];
    mn = min(mn, v);
    mx = max(mx, v);
  }
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
  if (lane == 0) {
    red[0][w] = mn;
    red[1][w] = mx;
  }
  __syncthreads();
  mn = red[0][0];
  mx = red[1][0];
  for (int j = 1; j < 16; ++j) {
    mn = min(mn, red[0][j]);
    mx = max(mx, red[1][j]);
  }
  uint32_t prefix = mn;
  if (mn != mx) {
    int hb = 31 - __clz(mn ^ mx);  // highest differing bit
    prefix = mn & ~((hb == 31) ? 0xFFFFFFFFu : ((2u << hb) - 1u));
    while (true) {
      const int shift = max(hb - 10, 0);
      const int width = hb - shift + 1;
      const uint32_t dmask = (1u << width) - 1u;
      const int above = shift + width;  // bits >= above must equal prefix's
      hist[t] = 0;
      hist[t + 1024] = 0;
      __syncthreads();
      for (int i = t; i < n; i += 1024) {
        const uint32_t v = u[i];
        const bool match = above >= 32 ? true : ((v >> above) == (prefix >> above));
        if (match) atomicAdd(&hist[(v >> shift) & dmask], 1);
      }
      __syncthreads();
      const int c0 = hist[2 * t], c1 = hist[2 * t + 1];
      int tot;
      const int pre = block_excl_scan_1024<int>(c0 + c1, wsum, tot);
      if (pre < k && k <= pre + c0) {
        sel_bin = 2 * t;
        sel_pos = pre;
      } else if (pre + c0 < k && k <= pre + c0 + c1) {
        sel_bin = 2 * t + 1;
        sel_pos = pre + c0;
      }
      __syncthreads();
      k -= sel_pos;
      prefix |= uint32_t(sel_bin) << shift;
      __syncthreads();
      if (shift == 0) break;
      hb = shift - 1;
    }
  }
  // ties: the k-th position (in order) holding key == prefix
  int running = 0;
  for (int base = 0; base < n; base += 1024) {
    const int i = base + t;
    const int f = (i < n && u[i] == prefix) ? 1 : 0;
    int tot;
    const int pre = block_excl_scan_1024<int>(f, wsum, tot);
    if (f && running + pre + 1 == k) sel_pos = sg.x + i;
    running += tot;
    __syncthreads();
    if (running >= k) break;
  }
  __syncthreads();
  if (t == 0) thr[size_t(h) * max_seg + blockIdx.x] = make_uint2(prefix, uint32_t(sel_pos));
}

__device__ __forceinline__ bool is_left(uint32_t key, int pos, uint2 th) {
  return key < th.x || (key == th.x && pos <= int(th.y));
}

// ---------------------------------------------------------------------------
// sums of both sides per chunk
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void sums_kernel(const T* __restrict__ x,
                                                   const int32_t* __restrict__ perm,
                                                   const uint32_t* __restrict__ keys,
                                                   const int4* __restrict__ chunks,
                                                   const uint2* __restrict__ thr, int max_seg,
                                                   int max_chunk, int N, float* __restrict__ part) {
  using G = RowGeo<T, D>;
  __shared__ float ws[4][2][D];
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 ch = chunks[blockIdx.x];
  const uint2 th = thr[size_t(h) * max_seg + ch.x];
  const int32_t* ph = perm + size_t(h) * N;
  const uint32_t* kh = keys + size_t(h) * N;
  const T* xh = x + size_t(h) * N * D;
  const int lane = t & 63, w = t >> 6;
  const int sub = lane % G::LPR, rsub = lane / G::LPR;
  float sl[G::EPV], sr[G::EPV];
#pragma unroll
  for (int e = 0; e < G::EPV; ++e) sl[e] = sr[e] = 0.f;
  for (int rb = w * G::RPW; rb < ch.z; rb += 4 * G::RPW) {
    const int r = rb + rsub;
    if (r < ch.z) {
      const int p = ch.y + r;
      float v[G::EPV];
      load_vec<T, G::EPV>(xh + size_t(ph[p]) * D + sub * G::EPV, v);
      if (is_left(kh[p], p, th)) {
#pragma unroll
        for (int e = 0; e < G::EPV; ++e) sl[e] += v[e];
      } else {
#pragma unroll
        for (int e = 0; e < G::EPV; ++e) sr[e] += v[e];
      }
    }
  }
  // combine the row groups of the wave (lanes with the same slice), fixed order
#pragma unroll
  for (int o = G::LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) {
      sl[e] += __shfl_xor(sl[e], o, 64);
      sr[e] += __shfl_xor(sr[e], o, 64);
    }
  }
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) {
      ws[w][0][sub * G::EPV + e] = sl[e];
      ws[w][1][sub * G::EPV + e] = sr[e];
    }
  }
  __syncthreads();
  float* out = part + (size_t(h) * max_chunk + blockIdx.x) * 2 * D;
  for (int i = t; i < 2 * D; i += 256) {
    const int s = i / D, c = i % D;
    out[i] = ((ws[0][s][c] + ws[1][s][c]) + ws[2][s][c]) + ws[3][s][c];
  }
}

template <int D>
__global__ __launch_bounds__(D) void update_kernel(const int4* __restrict__ segs,
                                                   const float* __restrict__ part, int max_seg,
                                                   int max_chunk, float* __restrict__ cen) {
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 sg = segs[blockIdx.x];
  if (sg.z == 0) return;
  const int nch = ceil_div(sg.y, BCH);
  float L = 0.f, R = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float* p = part + (size_t(h) * max_chunk + sg.w + c) * 2 * D;
    L += p[t];
    R += p[D + t];
  }
  float* o = cen + (size_t(h) * max_seg + blockIdx.x) * 2 * D;
  o[t] = L / float(sg.z);
  o[D + t] = R / float(sg.y - sg.z);
}

// ---------------------------------------------------------------------------
// stable partition
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void partition_kernel(const int32_t* __restrict__ perm_in,
                                                         int32_t* __restrict__ perm_out,
                                                         const uint32_t* __restrict__ keys,
                                                         const int4* __restrict__ segs,
                                                         const uint2* __restrict__ thr, int max_seg,
                                                         int N) {
  __shared__ int wsum[16];
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 sg = segs[blockIdx.x];
  const int32_t* pi = perm_in + size_t(h) * N;
  int32_t* po = perm_out + size_t(h) * N;
  if (sg.z == 0) {
    for (int i = t; i < sg.y; i += 1024) po[sg.x + i] = pi[sg.x + i];
    return;
  }
  const uint2 th = thr[size_t(h) * max_seg + blockIdx.x];
  const uint32_t* kh = keys + size_t(h) * N;
  int run_left = 0;
  for (int base = 0; base < sg.y; base += 1024) {
    const int i = base + t;
    const bool valid = i < sg.y;
    const int p = sg.x + i;
    const int left = (valid && is_left(kh[p], p, th)) ? 1 : 0;
    int tot;
    const int lpre = block_excl_scan_1024<int>(left, wsum, tot) + run_left;
    if (valid) {
      const int np = left ? sg.x + lpre : sg.x + sg.z + (i - lpre);
      po[np] = pi[p];
    }
    run_left += tot;
  }
}

__global__ void leaf_offsets_kernel(int32_t* off, int H, int C, int N, int L) {
  const int h = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c <= C) off[size_t(h) * (C + 1) + c] = min(c * L, N);
}

template <typename T, int D>
hipError_t run_levels(const void* xv, int H, int N, int L, int iters, const TreePlan& P, int4* segs,
                      int4* chunks, int32_t* pa, int32_t* pb, uint32_t* keys, float* cen,
                      uint2* thr, float* part, int32_t** final_perm, hipStream_t st) {
  const T* x = (const T*)xv;
  for (int lv = 0; lv < P.t.nlev; ++lv) {
    const int4* sg = segs + P.t.sb[lv];
    const int4* ck = chunks + P.t.cb[lv];
    const dim3 gs(P.t.nseg[lv], H), gc(P.t.nchunk[lv], H);
    for (int it = 0; it < iters; ++it) {
      delta_kernel<T, D><<<gc, 256, 0, st>>>(x, pa, sg, ck, cen, P.max_seg, N, it == 0, keys);
      select_kernel<<<gs, 1024, 0, st>>>(keys, sg, P.max_seg, N, thr);
      if (it + 1 < iters) {
        sums_kernel<T, D><<<gc, 256, 0, st>>>(x, pa, keys, ck, thr, P.max_seg, P.max_chunk, N, part);
        update_kernel<D><<<gs, D, 0, st>>>(sg, part, P.max_seg, P.max_chunk, cen);
      }
    }
    partition_kernel<<<gs, 1024, 0, st>>>(pa, pb, keys, sg, thr, P.max_seg, N);
    int32_t* tmp = pa;
    pa = pb;
    pb = tmp;
  }
  *final_perm = pa;
  return hipGetLastError();
}

}  // namespace

size_t bisect_scratch(int H, int N, int d, int leaf) {
  const TreePlan P = plan_tree(N, leaf);
  Arena a{nullptr, 0, 0};
  a.get<int4>(size_t(max(P.total_seg, 1)));
  a.get<int4>(size_t(max(P.total_chunk, 1)));
  a.get<int32_t>(size_t(H) * N);  // ping
  a.get<int32_t>(size_t(H) * N);  // pong
  a.get<uint32_t>(size_t(H) * N);  // keys
  a.get<float>(size_t(H) * max(P.max_seg, 1) * 2 * d);
  a.get<uint2>(size_t(H) * max(P.max_seg, 1));
  a.get<float>(size_t(H) * max(P.max_chunk, 1) * 2 * d);
  return a.used;
}

hipError_t bisect_run(const void* x, int dtype, int H, int N, int d, int leaf, int iters,
                      int32_t* perm_out, int32_t* offsets_out, Arena& s, hipStream_t st) {
  const TreePlan P = plan_tree(N, leaf);
  int4* segs = s.get<int4>(size_t(max(P.total_seg, 1)));
  int4* chunks = s.get<int4>(size_t(max(P.total_chunk, 1)));
  int32_t* other = s.get<int32_t>(size_t(H) * N);
  (void)s.get<int32_t>(size_t(H) * N);
  uint32_t* keys = s.get<uint32_t>(size_t(H) * N);
  float* cen = s.get<float>(size_t(H) * max(P.max_seg, 1) * 2 * d);
  uint2* thr = s.get<uint2>(size_t(H) * max(P.max_seg, 1));
  float* part = s.get<float>(size_t(H) * max(P.max_chunk, 1) * 2 * d);
  // ping-pong so that the last level writes perm_out
  int32_t* pa = (P.t.nlev % 2 == 0) ? perm_out : other;
  int32_t* pb = (P.t.nlev % 2 == 0) ? other : perm_out;
  iota_kernel<<<dim3(ceil_div(N, 256), H), 256, 0, st>>>(pa, N);
  int32_t* fin = pa;
  hipError_t e = hipSuccess;
  if (P.t.nlev > 0) {
    build_tree_kernel<<<1, 1024, 0, st>>>(P.t, N, leaf, segs, chunks);
    if (dtype == SA_F32 && d == 64)
      e = run_levels<float, 64>(x, H, N, leaf, iters, P, segs, chunks, pa, pb, keys, cen, thr, part, &fin, st);
    else if (dtype == SA_F32 && d == 128)
      e = run_levels<float, 128>(x, H, N, leaf, iters, P, segs, chunks, pa, pb, keys, cen, thr, part, &fin, st);
    else if (dtype == SA_BF16 && d == 64)
      e = run_levels<bf16_t, 64>(x, H, N, leaf, iters, P, segs, chunks, pa, pb, keys, cen, thr, part, &fin, st);
    else
      e = run_levels<bf16_t, 128>(x, H, N, leaf, iters, P, segs, chunks, pa, pb, keys, cen, thr, part, &fin, st);
  }
  if (e != hipSuccess) return e;
  if (fin != perm_out) return hipErrorUnknown;  // ping-pong parity is fixed above
  const int C = ceil_div(N, leaf);
  leaf_offsets_kernel<<<dim3(ceil_div(C + 1, 256), H), 256, 0, st>>>(offsets_out, H, C, N, leaf);
  return hipGetLastError();
}

}  // namespace sa
