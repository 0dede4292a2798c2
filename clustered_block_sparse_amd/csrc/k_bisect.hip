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
// segments per level.  Two phases:
//  * top phase (segments of more than SUB_N tokens), one level at a time for
//    all heads:
//      delta  : chunked, 16-byte slice per lane, sortable fp32 key per token;
//               the segment's key min / max is folded in with integer atomics
//      select : one workgroup per segment, exact k-th smallest (key, position)
//               via an interpolated histogram, then an LDS radix search
//      sums   : round 0 sums both sides; later rounds only re-read the tokens
//               that switched side (the sums change by exactly those rows);
//               per-chunk partials, added in chunk order per segment (fixed
//               order, no float atomics)
//      part.  : per segment ordered scan -> stable partition of positions
//      next   : a level's last delta pass also forms its children's
//               first-round keys under a prediction of their first two
//               tokens; the partition checks it, and a verified child skips
//               its first delta pass (results identical either way)
//    The passes that read every row (delta, the first round's sums)
//    alternate the order in which their workgroups walk the heads and
//    chunks, so a pass starts on the rows the previous one read last, which
//    the memory-side cache still holds (each block writes the same outputs
//    either way).
//  * subtree phase: one workgroup finishes each segment of at most SUB_N
//    tokens through all remaining levels, with positions, keys and sides in
//    LDS and rows re-read through the caches (four rows in flight per lane).

#include <algorithm>
#include <vector>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int BCH = 1024;    // positions per chunk (top phase)
constexpr int DELTA_SPLIT = 4;  // delta pass: workgroups per chunk
constexpr int SUB_N = 2560;  // segments up to this many tokens finish in one workgroup
constexpr int MAXLEV = 32;
constexpr int SUB_THREADS = 512;

struct LevelTabs {
  int nlev;  // top levels; the final segment list is level nlev
  int nseg[MAXLEV + 1], nchunk[MAXLEV], sb[MAXLEV + 1], cb[MAXLEV];
  int L, subn;
};

struct TreePlan {
  LevelTabs t;
  int total_seg, total_chunk, max_seg, max_chunk;
};

__host__ __device__ inline bool is_active(int n, int L, int subn) {
  return ceil_div(n, L) >= 2 && n > subn;
}

TreePlan plan_tree(int N, int L, int subn) {
  TreePlan p{};
  p.t.L = L;
  p.t.subn = subn;
  std::vector<int> st{0}, nn{N};
  while (p.t.nlev < MAXLEV) {
    bool any = false;
    for (int n : nn)
      if (is_active(n, L, subn)) any = true;
    if (!any) break;
    const int lv = p.t.nlev++;
    p.t.nseg[lv] = int(nn.size());
    p.t.sb[lv] = p.total_seg;
    p.total_seg += int(nn.size());
    int nch = 0;
    std::vector<int> st2, nn2;
    for (size_t k = 0; k < nn.size(); ++k) {
      if (is_active(nn[k], L, subn)) {
        const int nl = L * ceil_div(ceil_div(nn[k], L), 2);
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
  p.t.nseg[p.t.nlev] = int(nn.size());
  p.t.sb[p.t.nlev] = p.total_seg;
  p.total_seg += int(nn.size());
  p.max_seg = max(p.max_seg, 1);
  p.max_chunk = max(p.max_chunk, 1);
  return p;
}

// ---------------------------------------------------------------------------
// block helpers
// ---------------------------------------------------------------------------
// exclusive scan over the block (blockDim a multiple of 64, <= 1024)
template <typename V>
__device__ V block_excl_scan(V v, V* wsum /*[16]*/, V& total) {
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

__device__ __forceinline__ bool is_left(uint32_t key, int pos, uint2 th) {
  return key < th.x || (key == th.x && pos <= int(th.y));
}

// Exact k-th smallest (1-based) of (key[i], i) over i < n: keys read through
// `get`.  A radix search over 11-bit digits below the common prefix of the
// minimum and maximum key, then an ordered scan over indices for the tie.
// All threads of the block call it; the result is (key, index).
struct SelectShared {
  int hist[2048];
  int wsum[16];
  uint32_t red[2][16];
  int sel_bin, sel_pos;
};

template <typename Get>
__device__ uint2 block_select(Get get, int n, int k, SelectShared& sh) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nt = blockDim.x, nw = nt >> 6;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = t; i < n; i += nt) {
    const uint32_t v = get(i);
    mn = min(mn, v);
    mx = max(mx, v);
  }
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
  if (lane == 0) {
    sh.red[0][w] = mn;
    sh.red[1][w] = mx;
  }
  __syncthreads();
  mn = sh.red[0][0];
  mx = sh.red[1][0];
  for (int j = 1; j < nw; ++j) {
    mn = min(mn, sh.red[0][j]);
    mx = max(mx, sh.red[1][j]);
  }
  __syncthreads();
  uint32_t prefix = mn;
  if (mn != mx) {
    int hb = 31 - __clz(mn ^ mx);
    prefix = hb == 31 ? 0u : (mn & ~((2u << hb) - 1u));
    while (true) {
      const int shift = max(hb - 10, 0);
      const int width = hb - shift + 1;
      const uint32_t dmask = (1u << width) - 1u;
      const int above = shift + width;
      for (int b = t; b < 2048; b += nt) sh.hist[b] = 0;
      __syncthreads();
      for (int i = t; i < n; i += nt) {
        const uint32_t v = get(i);
        const bool match = above >= 32 ? true : ((v >> above) == (prefix >> above));
        if (match) atomicAdd(&sh.hist[(v >> shift) & dmask], 1);
      }
      __syncthreads();
      // bins per thread: 2048 / nt
      const int bpt = 2048 / nt;
      int loc = 0;
      for (int b = 0; b < bpt; ++b) loc += sh.hist[t * bpt + b];
      int tot;
      int pre = block_excl_scan<int>(loc, sh.wsum, tot);
      if (pre < k && k <= pre + loc) {
        for (int b = 0; b < bpt; ++b) {
          const int c = sh.hist[t * bpt + b];
          if (pre < k && k <= pre + c) {
            sh.sel_bin = t * bpt + b;
            sh.sel_pos = pre;
          }
          pre += c;
        }
      }
      __syncthreads();
      k -= sh.sel_pos;
      prefix |= uint32_t(sh.sel_bin) << shift;
      __syncthreads();
      if (shift == 0) break;
      hb = shift - 1;
    }
  }
  int running = 0;
  for (int base = 0; base < n; base += nt) {
    const int i = base + t;
    const int f = (i < n && get(i) == prefix) ? 1 : 0;
    int tot;
    const int pre = block_excl_scan<int>(f, sh.wsum, tot);
    if (f && running + pre + 1 == k) sh.sel_pos = i;
    running += tot;
    __syncthreads();
    if (running >= k) break;
  }
  __syncthreads();
  const uint2 r = make_uint2(prefix, uint32_t(sh.sel_pos));
  __syncthreads();
  return r;
}

// k-th smallest (1-based) of m distinct 64-bit keys held in LDS: radix search
// over 11-bit digits below the common prefix of the minimum and maximum.
struct Sel64Shared {
  int hist[2048];
  int wsum[16];
  unsigned long long red[2][16];
  int sel_bin, sel_pos;
};

__device__ unsigned long long lds_select64(const unsigned long long* key, int m, int k, Sel64Shared& sh) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nt = blockDim.x, nw = nt >> 6;
  unsigned long long mn = ~0ull, mx = 0ull;
  for (int i = t; i < m; i += nt) {
    const unsigned long long v = key[i];
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long a = __shfl_xor(mn, o, 64), c = __shfl_xor(mx, o, 64);
    mn = a < mn ? a : mn;
    mx = c > mx ? c : mx;
  }
  if (lane == 0) {
    sh.red[0][w] = mn;
    sh.red[1][w] = mx;
  }
  __syncthreads();
  mn = sh.red[0][0];
  mx = sh.red[1][0];
  for (int j = 1; j < nw; ++j) {
    mn = sh.red[0][j] < mn ? sh.red[0][j] : mn;
    mx = sh.red[1][j] > mx ? sh.red[1][j] : mx;
  }
  __syncthreads();
  if (mn == mx) return mn;
  int hb = 63 - __clzll(mn ^ mx);
  unsigned long long prefix = hb == 63 ? 0ull : (mn & ~((2ull << hb) - 1ull));
  while (true) {
    const int shift = max(hb - 10, 0);
    const int width = hb - shift + 1;
    const unsigned long long dmask = (1ull << width) - 1ull;
    const int above = shift + width;
    for (int b = t; b < 2048; b += nt) sh.hist[b] = 0;
    __syncthreads();
    for (int i = t; i < m; i += nt) {
      const unsigned long long v = key[i];
      const bool match = above >= 64 ? true : ((v >> above) == (prefix >> above));
      if (match) atomicAdd(&sh.hist[int((v >> shift) & dmask)], 1);
    }
    __syncthreads();
    const int bpt = 2048 / nt;
    int loc = 0;
    for (int b = 0; b < bpt; ++b) loc += sh.hist[t * bpt + b];
    int tot;
    int pre = block_excl_scan<int>(loc, sh.wsum, tot);
    if (pre < k && k <= pre + loc) {
      for (int b = 0; b < bpt; ++b) {
        const int c = sh.hist[t * bpt + b];
        if (pre < k && k <= pre + c) {
          sh.sel_bin = t * bpt + b;
          sh.sel_pos = pre;
        }
        pre += c;
      }
    }
    __syncthreads();
    k -= sh.sel_pos;
    prefix |= (unsigned long long)sh.sel_bin << shift;
    __syncthreads();
    if (shift == 0) break;
    hb = shift - 1;
  }
  return prefix;
}

// ---------------------------------------------------------------------------
// tree tables on the device (one workgroup of 1024 threads)
// segs: int4 {start, n, n_left (0 = not split at this level), first chunk}
// chunks: int4 {segment (level-local), position, count, 0}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tree_kernel(LevelTabs tb, int N, int4* segs,
                                                          int4* chunks, int32_t* kids) {
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  if (t == 0) segs[0] = make_int4(0, N, 0, 0);
  __threadfence_block();
  __syncthreads();
  for (int lv = 0; lv < tb.nlev; ++lv) {
    int chunk_carry = 0, child_carry = 0;
    for (int base = 0; base < tb.nseg[lv]; base += 1024) {
      const int k = base + t;
      int4 s = make_int4(0, 0, 0, 0);
      int nchunk = 0, nchild = 0, nl = 0;
      if (k < tb.nseg[lv]) {
        s = segs[tb.sb[lv] + k];
        if (is_active(s.y, tb.L, tb.subn)) {
          nl = tb.L * ceil_div(ceil_div(s.y, tb.L), 2);
          nchunk = ceil_div(s.y, BCH);
          nchild = 2;
        } else {
          nchild = 1;
        }
      }
      int tot1, tot2;
      const int cpre = block_excl_scan<int>(nchunk, wsum, tot1) + chunk_carry;
      const int kpre = block_excl_scan<int>(nchild, wsum, tot2) + child_carry;
      if (k < tb.nseg[lv]) {
        segs[tb.sb[lv] + k] = make_int4(s.x, s.y, nl, cpre);
        kids[tb.sb[lv] + k] = kpre;  // index of its first child one level down
        for (int c = 0; c < nchunk; ++c) {
          const int pos = s.x + c * BCH;
          chunks[tb.cb[lv] + cpre + c] = make_int4(k, pos, min(BCH, s.x + s.y - pos), 0);
        }
        int4* nxt = segs + tb.sb[lv + 1] + kpre;
        if (nchild == 2) {
          nxt[0] = make_int4(s.x, nl, 0, 0);
          nxt[1] = make_int4(s.x + nl, s.y - nl, 0, 0);
        } else {
          nxt[0] = make_int4(s.x, s.y, 0, 0);
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

__global__ void init_minmax(uint2* p, size_t n) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = make_uint2(0xFFFFFFFFu, 0u);
}

__global__ void zero_i32(int32_t* p, size_t n) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// row geometry: one 16-byte vector per lane, LPR lanes per row
// ---------------------------------------------------------------------------
template <typename T, int D>
struct RowGeo {
  static constexpr int EPV = 16 / int(sizeof(T));  // elements per 16-byte vector
  static constexpr int LPR = D / EPV;              // lanes per row
  static constexpr int RPW = 64 / LPR;             // rows per wave step
};

// Sum over each aligned group of LPR lanes (every lane gets it) by DPP moves
// inside 16-lane rows: quad_perm [1,0,3,2] and [2,3,0,1], then the half-row
// and row mirrors (a shuffle would go through the LDS crossbar); groups wider
// than a row add the rows by shuffles.
template <int DPPC>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), DPPC, 0xF, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (LPR >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (LPR >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <typename T, int EPV>
__device__ __forceinline__ void unpack_vec(uint4 u, float (&v)[EPV]) {
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

template <typename T>
__device__ __forceinline__ uint4 ld16(const T* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Rows of head h.  Two tensors of the same shape can be bisected together as
// one problem of H0 + H1 heads: heads below h0 are those of x0, the others
// those of x1, so every launch covers both.
template <typename T>
struct Src2 {
  const T* x0;
  const T* x1;
  int h0;
  __device__ __forceinline__ const T* head(int h, int N, int D) const {
    return h < h0 ? x0 + size_t(h) * N * D : x1 + size_t(h - h0) * N * D;
  }
};

// Optional outputs of the subtree phase: every head's rows in cluster order
// and its leaf (cluster) means, split between two tensors like Src2.
template <typename T>
struct LeafOut {
  T* xp0;
  T* xp1;
  float* c0;
  float* c1;
  int C;  // leaves per head
};

// ---------------------------------------------------------------------------
// top phase kernels (grid.y = heads)
// ---------------------------------------------------------------------------
constexpr int NBIN = 2048;      // interpolated histogram bins of a segment's keys
constexpr int CAND_CAP = 4096;  // candidates of the selected bin kept per segment

struct TopBufs {
  const int4* segs;    // level table
  const int4* chunks;  // level chunk table
  int32_t* perm;       // [H][N] current order
  uint32_t* keys;      // [H][N]
  uint8_t* side;       // [H][N] 1 = left in the previous round
  float* cen;          // [H][max_seg][2][D]  means of the two sides
  float* ssum;         // [H][max_seg][2][D]  sums of the two sides
  uint2* thr;          // [H][max_seg]
  float* part;         // [H][max_chunk][2][D]
  uint2* segmm;        // [H][max_seg] min / max key of the round (reset after use)
  int32_t* ghist;      // [H][max_seg][NBIN] key histogram of the round (zero between uses)
  int2* selbin;        // [H][max_seg] bin holding rank n_left, rank inside it (bin -1: keys all equal)
  unsigned long long* cand;  // [H][max_seg][CAND_CAP] (key << 32 | position) of that bin
  int32_t* ccount;     // [H][max_seg] candidates (zero between uses)
  // children's first round formed during the parent's last one (see
  // predict_children below)
  const int32_t* kids; // level table: index of each segment's first child one level down
  int4* pred;          // [H][max_seg] predicted first two left / right positions (-1: none)
  uint32_t* keyL;      // [H][N] round-0 key of each row for the predicted left child
  uint32_t* keyR;      // [H][N] ... for the predicted right child
  uint32_t* keys_next; // [H][N] children's round-0 keys, in the children's order
  int32_t* pred_ok;    // [H][max_seg] (next level) 1: the child's round-0 keys are in place
  // A child's total is its side's sum in the parent's final split, so its
  // first round sums only its right side (never the larger one) and takes
  // the left as total - right.
  float* ctot;         // [H][max_seg][D] total of each segment of the level (from its parent)
  int tot_out;         // the partition writes the children's totals
  int d;
  int max_seg, max_chunk, N, round;  // round: 0 = first round of a level
  int rev;  // full passes over the rows: walk the blocks in reverse order
};

// A child segment starts its first round from its first two tokens, which
// are the first two positions (in the parent's order) of its side of the
// parent's final split.  Before the parent's last round they are predicted
// from the sides of the round before; the last round's delta pass then also
// forms, for every row, the child's first-round key under that prediction
// (the same arithmetic, in the same order, as the child's own pass), and the
// partition carries the keys of each row's side into the children's order
// and checks the prediction against the actual first positions.  A child
// whose prediction held skips its first delta pass; the others run it.
__global__ __launch_bounds__(64) void firsts_kernel(TopBufs b) {
  const int h = blockIdx.y, lane = threadIdx.x;
  const int4 sg = b.segs[blockIdx.x];
  if (sg.z == 0) return;
  const uint8_t* sd = b.side + size_t(h) * b.N + sg.x;
  int fl0 = -1, fl1 = -1, fr0 = -1, fr1 = -1, nl = 0, nr = 0;
  for (int base = 0; base < sg.y && (nl < 2 || nr < 2); base += 64) {
    const int i = base + lane;
    const bool v = i < sg.y;
    const bool left = v && sd[i] != 0;
    uint64_t ml = __ballot(left), mr = __ballot(v && !left);
    while (nl < 2 && ml) {
      const int p = sg.x + base + __ffsll((unsigned long long)ml) - 1;
      if (nl == 0) fl0 = p; else fl1 = p;
      ++nl;
      ml &= ml - 1;
    }
    while (nr < 2 && mr) {
      const int p = sg.x + base + __ffsll((unsigned long long)mr) - 1;
      if (nr == 0) fr0 = p; else fr1 = p;
      ++nr;
      mr &= mr - 1;
    }
  }
  if (lane == 0)
    b.pred[size_t(h) * b.max_seg + blockIdx.x] =
        make_int4(nl == 2 ? fl0 : -1, nl == 2 ? fl1 : -1, nr == 2 ? fr0 : -1, nr == 2 ? fr1 : -1);
}

// PRED: also the predicted children's first-round keys of every row.
// use_ok: a segment whose first-round keys (and their min / max) its parent
// already formed has nothing to do.
template <typename T, int D, bool PRED>
__global__ __launch_bounds__(256) void delta_kernel(Src2<T> x, TopBufs b, int first, int use_ok) {
  using G = RowGeo<T, D>;
  constexpr int U = PRED ? 4 : 8;  // wave steps in flight (three dot products per row in PRED)
  __shared__ float wv[D], mv[D];
  __shared__ float wvc[PRED ? 2 : 1][D], mvc[PRED ? 2 : 1][D];  // children (left, right)
  __shared__ int pidx[BCH / DELTA_SPLIT];  // the part's rows (original tokens)
  const int bx = b.rev ? int(gridDim.x) - 1 - int(blockIdx.x) : int(blockIdx.x);
  const int h = b.rev ? int(gridDim.y) - 1 - int(blockIdx.y) : int(blockIdx.y), t = threadIdx.x;
  // a workgroup takes one of the DELTA_SPLIT equal parts of a chunk: more,
  // shorter workgroups keep the last wave of the launch from idling the chip
  const int4 chunk = b.chunks[bx / DELTA_SPLIT];
  const int r0 = (bx % DELTA_SPLIT) * (BCH / DELTA_SPLIT);
  if (r0 >= chunk.z) return;
  const int4 ch = make_int4(chunk.x, chunk.y + r0, min(BCH / DELTA_SPLIT, chunk.z - r0), chunk.w);
  const int lane = t & 63, w = t >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (use_ok && b.pred_ok[size_t(h) * b.max_seg + ch.x]) return;
  {
    const int4 sg = b.segs[ch.x];
    const int32_t* ph = b.perm + size_t(h) * b.N;
    const T* __restrict__ xh = x.head(h, b.N, D);
    for (int i = t; i < ch.z; i += 256) pidx[i] = ph[ch.y + i];
    if (t < D) {
      float c1, c2;
      if (first) {
        c1 = to_f(xh[size_t(ph[sg.x]) * D + t]);
        c2 = to_f(xh[size_t(ph[sg.x + 1]) * D + t]);
      } else {
        const float* c = b.cen + (size_t(h) * b.max_seg + ch.x) * 2 * D;
        c1 = c[t];
        c2 = c[D + t];
      }
      wv[t] = c2 - c1;
      mv[t] = c1 + c2;
      if constexpr (PRED) {
        // a child without a prediction gets zero centroids (its keys go unused)
        const int4 pr = b.pred[size_t(h) * b.max_seg + ch.x];
        float a1 = 0.f, a2 = 0.f, q1 = 0.f, q2 = 0.f;
        if (pr.x >= 0) {
          a1 = to_f(xh[size_t(ph[pr.x]) * D + t]);
          a2 = to_f(xh[size_t(ph[pr.y]) * D + t]);
        }
        if (pr.z >= 0) {
          q1 = to_f(xh[size_t(ph[pr.z]) * D + t]);
          q2 = to_f(xh[size_t(ph[pr.w]) * D + t]);
        }
        wvc[0][t] = a2 - a1;
        mvc[0][t] = a1 + a2;
        wvc[PRED ? 1 : 0][t] = q2 - q1;
        mvc[PRED ? 1 : 0][t] = q1 + q2;
      }
    }
    __syncthreads();
    const int sub = lane % G::LPR, rsub = lane / G::LPR;
    float wr[G::EPV], mr[G::EPV];
    float wl[PRED ? G::EPV : 1], ml[PRED ? G::EPV : 1], wq[PRED ? G::EPV : 1], mq[PRED ? G::EPV : 1];
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) {
      wr[e] = wv[sub * G::EPV + e];
      mr[e] = mv[sub * G::EPV + e];
      if constexpr (PRED) {
        wl[e] = wvc[0][sub * G::EPV + e];
        ml[e] = mvc[0][sub * G::EPV + e];
        wq[e] = wvc[PRED ? 1 : 0][sub * G::EPV + e];
        mq[e] = mvc[PRED ? 1 : 0][sub * G::EPV + e];
      }
    }
    // delta = sum w (2 x - m) = 2 (w . x) - w . m: the lane's share of w . m
    // is a constant of the round, so each element costs one FMA per key
    float cr = 0.f, cl = 0.f, cq = 0.f;
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) {
      cr = fmaf(wr[e], mr[e], cr);
      if constexpr (PRED) {
        cl = fmaf(wl[e], ml[e], cl);
        cq = fmaf(wq[e], mq[e], cq);
      }
    }
    constexpr int STEP = 4 * G::RPW;  // rows per block step
    for (int rb = w * G::RPW; rb < ch.z; rb += U * STEP) {
      int pos[U];
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rb + u * STEP + rsub;
        pos[u] = r < ch.z ? r : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = ld16(xh + size_t(pidx[pos[u]]) * D + sub * G::EPV);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[G::EPV];
        unpack_vec<T, G::EPV>(raw[u], v);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < G::EPV; ++e) acc = fmaf(wr[e], v[e], acc);
        acc = fmaf(2.f, acc, -cr);
        acc = row_sum<G::LPR>(acc);
        const int r = rb + u * STEP + rsub;
        const uint32_t key = sortable(acc);
        if (r < ch.z) {
          kmin = min(kmin, key);
          kmax = max(kmax, key);
          if (sub == 0) b.keys[size_t(h) * b.N + ch.y + pos[u]] = key;
        }
        if constexpr (PRED) {
          float al = 0.f, aq = 0.f;
#pragma unroll
          for (int e = 0; e < G::EPV; ++e) {
            al = fmaf(wl[e], v[e], al);
            aq = fmaf(wq[e], v[e], aq);
          }
          al = fmaf(2.f, al, -cl);
          aq = fmaf(2.f, aq, -cq);
          al = row_sum<G::LPR>(al);
          aq = row_sum<G::LPR>(aq);
          if (r < ch.z && sub == 0) {
            b.keyL[size_t(h) * b.N + ch.y + pos[u]] = sortable(al);
            b.keyR[size_t(h) * b.N + ch.y + pos[u]] = sortable(aq);
          }
        }
      }
    }
  }
  // chunk min / max -> segment (integer atomics: order independent)
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  __shared__ uint32_t rmm[2][4];
  if (lane == 0) {
    rmm[0][w] = kmin;
    rmm[1][w] = kmax;
  }
  __syncthreads();
  if (t == 0) {
    const uint32_t a = min(min(rmm[0][0], rmm[0][1]), min(rmm[0][2], rmm[0][3]));
    const uint32_t c = max(max(rmm[1][0], rmm[1][1]), max(rmm[1][2], rmm[1][3]));
    uint2* mm = b.segmm + size_t(h) * b.max_seg + ch.x;
    atomicMin(&mm->x, a);
    atomicMax(&mm->y, c);
  }
}

// Exact (key, position) of rank n_left in every segment, in four launches
// that spread each segment over its chunks:
//   hist: per-chunk histograms of NBIN bins interpolated between the
//         segment's min / max key (folded in by the delta pass), added into
//         the segment's histogram (linear in the keys' float values: the
//         keys' own bits are close to logarithmic in |delta|, and a round
//         whose deltas take both signs would put a large share of the tokens
//         into the median's bin);
//   find: the bin holding rank n_left and the rank inside it;
//   cand: that bin's keys with their positions, as distinct 64-bit values;
//   pick: the exact rank among them (up to 1024: each thread counts the
//         candidates below its own; up to CAND_CAP: a radix search in LDS),
//         or, when the bin overflows CAND_CAP, a radix search over all of the
//         segment's keys.
// Only integer atomics are used; the selected (key, position) is unique, so
// the result does not depend on their order.
__device__ __forceinline__ float key_value(uint32_t k) {  // inverse of sortable()
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
// Bins of a segment's round, monotone in the key: (value - min) scaled to
// [0, NBIN) in fp64 (each step rounds monotonically), clamped.
struct BinMap {
  double lo, scale;
};
__device__ __forceinline__ BinMap bin_map(uint2 mm) {
  const double lo = key_value(mm.x), hi = key_value(mm.y);
  return BinMap{lo, hi > lo ? double(NBIN) / (hi - lo) : 0.0};
}
__device__ __forceinline__ int bin_of(uint32_t v, const BinMap& bm) {
  const int b = int((double(key_value(v)) - bm.lo) * bm.scale);
  return b < 0 ? 0 : (b < NBIN ? b : NBIN - 1);
}

__global__ __launch_bounds__(256) void hist_kernel(TopBufs b) {
  __shared__ int hist[NBIN];
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 ch = b.chunks[blockIdx.x];
  const size_t si = size_t(h) * b.max_seg + ch.x;
  const uint2 mm = b.segmm[si];
  if (mm.x == mm.y) return;
  for (int i = t; i < NBIN; i += 256) hist[i] = 0;
  __syncthreads();
  const uint32_t* u = b.keys + size_t(h) * b.N + ch.y;
  const BinMap bm = bin_map(mm);
  for (int i = t; i < ch.z; i += 256) atomicAdd(&hist[bin_of(u[i], bm)], 1);
  __syncthreads();
  int* g = b.ghist + si * NBIN;
  for (int i = t; i < NBIN; i += 256)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ __launch_bounds__(256) void find_kernel(TopBufs b) {
  __shared__ int wsum[16];
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 sg = b.segs[blockIdx.x];
  if (sg.z == 0) return;
  const size_t si = size_t(h) * b.max_seg + blockIdx.x;
  const uint2 mm = b.segmm[si];
  if (mm.x == mm.y) {
    if (t == 0) b.selbin[si] = make_int2(-1, 0);
    return;
  }
  constexpr int BPT = NBIN / 256;
  int* g = b.ghist + si * NBIN;
  int c[BPT], loc = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = g[t * BPT + j];
    loc += c[j];
  }
  int tot;
  int pre = block_excl_scan<int>(loc, wsum, tot);
  const int k = sg.z;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (pre < k && k <= pre + c[j]) b.selbin[si] = make_int2(t * BPT + j, k - pre);
    pre += c[j];
    g[t * BPT + j] = 0;  // ready for the next round
  }
}

__global__ __launch_bounds__(256) void cand_kernel(TopBufs b) {
  const int h = blockIdx.y, t = threadIdx.x, lane = t & 63;
  const int4 ch = b.chunks[blockIdx.x];
  const size_t si = size_t(h) * b.max_seg + ch.x;
  const int2 sb = b.selbin[si];
  if (sb.x < 0) return;
  const uint2 mm = b.segmm[si];
  const uint32_t* u = b.keys + size_t(h) * b.N + ch.y;
  unsigned long long* cd = b.cand + si * CAND_CAP;
  const BinMap bm = bin_map(mm);
  for (int i0 = 0; i0 < ch.z; i0 += 256) {
    const int i = i0 + t;
    const uint32_t v = i < ch.z ? u[i] : 0u;
    const bool f = i < ch.z && bin_of(v, bm) == sb.x;
    const uint64_t bal = __ballot(f);
    if (!bal) continue;
    const int lead = __ffsll((unsigned long long)bal) - 1;
    int base = 0;
    if (lane == lead) base = atomicAdd(&b.ccount[si], __popcll(bal));
    base = __shfl(base, lead, 64);
    const int slot = base + __popcll(bal & ((uint64_t(1) << lane) - 1));
    if (f && slot < CAND_CAP) cd[slot] = ((unsigned long long)v << 32) | uint32_t(ch.y + i);
  }
}

__global__ __launch_bounds__(1024) void pick_kernel(TopBufs b) {
  __shared__ unsigned long long cand[CAND_CAP];
  __shared__ Sel64Shared s64;
  __shared__ SelectShared gsh;
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 sg = b.segs[blockIdx.x];
  if (sg.z == 0) return;
  const size_t si = size_t(h) * b.max_seg + blockIdx.x;
  const uint2 mm = b.segmm[si];
  const int2 sb = b.selbin[si];
  const int m = sb.x < 0 ? 0 : b.ccount[si];
  __syncthreads();
  if (t == 0) {  // ready for the next round
    b.segmm[si] = make_uint2(0xFFFFFFFFu, 0u);
    b.ccount[si] = 0;
  }
  uint2 res;
  if (sb.x < 0) {
    res = make_uint2(mm.x, uint32_t(sg.x + sg.z - 1));  // all keys equal: rank k is position k-1
  } else if (m <= 1024) {
    // distinct values: the one with exactly sb.y - 1 smaller candidates
    const unsigned long long mine = t < m ? b.cand[si * CAND_CAP + t] : 0ull;
    if (t < m) cand[t] = mine;
    __syncthreads();
    int below = 0;
    for (int u = 0; u < m; ++u) below += cand[u] < mine ? 1 : 0;
    if (t < m && below == sb.y - 1) cand[CAND_CAP - 1] = mine;
    __syncthreads();
    const unsigned long long r = cand[CAND_CAP - 1];
    res = make_uint2(uint32_t(r >> 32), uint32_t(r & 0xFFFFFFFFull));
  } else if (m <= CAND_CAP) {
    for (int i = t; i < m; i += 1024) cand[i] = b.cand[si * CAND_CAP + i];
    __syncthreads();
    const unsigned long long r = lds_select64(cand, m, sb.y, s64);
    res = make_uint2(uint32_t(r >> 32), uint32_t(r & 0xFFFFFFFFull));
  } else {
    const uint32_t* u = b.keys + size_t(h) * b.N + sg.x;
    const uint2 r = block_select([&](int i) { return u[i]; }, sg.y, sg.z, gsh);
    res = make_uint2(r.x, r.y + sg.x);
  }
  if (t == 0) b.thr[si] = res;
}

// Sums of one chunk into its partial slot.  FULL (round 0): both sides from
// scratch.  Otherwise: the tokens whose side changed since the previous round,
// found with vectorised key/side reads and compacted in position order, give
// the change of the left sum; only their rows are read.  Sides are updated.
template <typename T, int D, bool FULL, bool RIGHT = false>
__global__ __launch_bounds__(256) void sums_kernel(Src2<T> x, TopBufs b) {
  using G = RowGeo<T, D>;
  constexpr int U = FULL ? 8 : 4;
  constexpr int STEP = 4 * G::RPW;
  __shared__ float ws[4][2][D];
  __shared__ int list[BCH];
  __shared__ int wsum[16];
  const int bx = b.rev ? int(gridDim.x) - 1 - int(blockIdx.x) : int(blockIdx.x);
  const int h = b.rev ? int(gridDim.y) - 1 - int(blockIdx.y) : int(blockIdx.y), t = threadIdx.x;
  const int4 ch = b.chunks[bx];
  const uint2 th = b.thr[size_t(h) * b.max_seg + ch.x];
  const int32_t* ph = b.perm + size_t(h) * b.N;
  const uint32_t* kh = b.keys + size_t(h) * b.N;
  uint8_t* sd = b.side + size_t(h) * b.N;
  const T* __restrict__ xh = x.head(h, b.N, D);
  const int lane = t & 63, w = t >> 6;
  const int sub = lane % G::LPR, rsub = lane / G::LPR;
  int cnt = ch.z;
  if constexpr (!FULL) {
    // four consecutive positions per thread (chunk starts are 4-aligned: leaf
    // and chunk sizes are multiples of 4)
    const int i0 = 4 * t;
    int sgn4[4] = {0, 0, 0, 0};
    int ns = 0;
    if (i0 < ch.z) {
      const int p0 = ch.y + i0;
      uint32_t kv[4];
      uint32_t sv = 0;
      if (i0 + 4 <= ch.z && (p0 & 3) == 0) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(kh + p0);
        kv[0] = k4.x; kv[1] = k4.y; kv[2] = k4.z; kv[3] = k4.w;
        sv = *reinterpret_cast<const uint32_t*>(sd + p0);
      } else {
        for (int q = 0; q < 4; ++q) {
          kv[q] = i0 + q < ch.z ? kh[p0 + q] : 0u;
          sv |= uint32_t(i0 + q < ch.z ? sd[p0 + q] : 0) << (8 * q);
        }
      }
      uint32_t nsv = sv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (i0 + q >= ch.z) break;
        const bool left = is_left(kv[q], p0 + q, th);
        const bool was = ((sv >> (8 * q)) & 0xFF) != 0;
        if (left != was) {
          sgn4[q] = left ? 1 : -1;
          ++ns;
          nsv = (nsv & ~(0xFFu << (8 * q))) | (uint32_t(left ? 1 : 0) << (8 * q));
        }
      }
      if (ns) {
        if (i0 + 4 <= ch.z && (p0 & 3) == 0) {
          *reinterpret_cast<uint32_t*>(sd + p0) = nsv;
        } else {
          for (int q = 0; q < 4 && i0 + q < ch.z; ++q) sd[p0 + q] = uint8_t((nsv >> (8 * q)) & 0xFF);
        }
      }
    }
    int tot;
    int pre = block_excl_scan<int>(ns, wsum, tot);
    for (int q = 0; q < 4; ++q)
      if (sgn4[q]) list[pre++] = sgn4[q] > 0 ? (ch.y + i0 + q) : ~(ch.y + i0 + q);
    cnt = tot;
    __syncthreads();
  }
  if constexpr (FULL && !RIGHT) {
    // the chunk's rows and sides, staged (sides are written here)
    for (int i = t; i < ch.z; i += 256) {
      const int p = ch.y + i;
      const bool left = is_left(kh[p], p, th);
      list[i] = left ? ph[p] : ~ph[p];
      sd[p] = left ? 1 : 0;
    }
    __syncthreads();
  }
  if constexpr (FULL && RIGHT) {
    // sides written for every row; only the right side's rows are listed
    // (in position order), the left side's sum follows from the total
    const int i0 = 4 * t;
    int nr = 0, tok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tok[q] = -1;
      const int i = i0 + q;
      if (i < ch.z) {
        const int p = ch.y + i;
        const bool left = is_left(kh[p], p, th);
        sd[p] = left ? 1 : 0;
        if (!left) {
          tok[q] = ph[p];
          ++nr;
        }
      }
    }
    int tot;
    int pre = block_excl_scan<int>(nr, wsum, tot);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (tok[q] >= 0) list[pre++] = ~tok[q];
    cnt = tot;
    __syncthreads();
  }
  float s0[G::EPV], s1[G::EPV];  // FULL: left, right.  Otherwise: change of left
#pragma unroll
  for (int e = 0; e < G::EPV; ++e) s0[e] = s1[e] = 0.f;
  for (int rb = w * G::RPW; rb < cnt; rb += U * STEP) {
    uint4 raw[U];
    int sgn[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * STEP + rsub;
      sgn[u] = 0;
      int p = 0;
      if (r < cnt) {
        const int e = list[r];
        if (FULL) {
          p = e >= 0 ? e : ~e;  // original token
          sgn[u] = e >= 0 ? 1 : 2;
        } else {
          p = ph[e >= 0 ? e : ~e];
          sgn[u] = e >= 0 ? 1 : -1;
        }
      }
      raw[u] = sgn[u] != 0 ? ld16(xh + size_t(p) * D + sub * G::EPV) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (sgn[u] == 0) continue;
      float v[G::EPV];
      unpack_vec<T, G::EPV>(raw[u], v);
      if (sgn[u] == 2) {
#pragma unroll
        for (int e = 0; e < G::EPV; ++e) s1[e] += v[e];
      } else if (sgn[u] == 1) {
#pragma unroll
        for (int e = 0; e < G::EPV; ++e) s0[e] += v[e];
      } else {
#pragma unroll
        for (int e = 0; e < G::EPV; ++e) s0[e] -= v[e];
      }
    }
  }
#pragma unroll
  for (int o = G::LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) {
      s0[e] += __shfl_xor(s0[e], o, 64);
      if constexpr (FULL) s1[e] += __shfl_xor(s1[e], o, 64);
    }
  }
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) {
      ws[w][0][sub * G::EPV + e] = s0[e];
      ws[w][1][sub * G::EPV + e] = FULL ? s1[e] : 0.f;
    }
  }
  __syncthreads();
  float* out = b.part + (size_t(h) * b.max_chunk + bx) * 2 * D;
  for (int i = t; i < 2 * D; i += 256) {
    const int sdx = i / D, c = i % D;
    out[i] = ((ws[0][sdx][c] + ws[1][sdx][c]) + ws[2][sdx][c]) + ws[3][sdx][c];
  }
}

// Per segment: partials in chunk order -> sums and means of the two sides.
template <int D, bool FULL, bool RIGHT = false>
__global__ __launch_bounds__(256) void update_kernel(TopBufs b) {
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 sg = b.segs[blockIdx.x];
  if (sg.z == 0) return;
  const int nch = ceil_div(sg.y, BCH);
  const size_t so = (size_t(h) * b.max_seg + blockIdx.x) * 2 * D;
  if constexpr (RIGHT) {
    // right side from the partials in chunk order, left = total - right
    const float* tt = b.ctot + (size_t(h) * b.max_seg + blockIdx.x) * D;
    for (int c = t; c < D; c += 256) {
      float r = 0.f;
      for (int q = 0; q < nch; ++q) r += b.part[(size_t(h) * b.max_chunk + sg.w + q) * 2 * D + D + c];
      const float l = tt[c] - r;
      b.ssum[so + c] = l;
      b.ssum[so + D + c] = r;
      b.cen[so + c] = l / float(sg.z);
      b.cen[so + D + c] = r / float(sg.y - sg.z);
    }
    return;
  }
  for (int i = t; i < 2 * D; i += 256) {
    const int sdx = i / D, c = i % D;
    const int src = FULL ? i : c;
    float acc = 0.f;
    for (int q = 0; q < nch; ++q) acc += b.part[(size_t(h) * b.max_chunk + sg.w + q) * 2 * D + src];
    const float tot = FULL ? acc : b.ssum[so + i] + (sdx == 0 ? acc : -acc);
    b.ssum[so + i] = tot;
    b.cen[so + i] = tot / float(sdx == 0 ? sg.z : sg.y - sg.z);
  }
}

// Stable partition of every split segment.  PRED: each row also carries its
// side's predicted first-round key into the children's order, the prediction
// of each child (its first two positions) is checked, and a child whose
// prediction held gets the min / max of its keys (for its first selection).
template <bool PRED>
__global__ __launch_bounds__(1024) void partition_kernel(TopBufs b, const int32_t* __restrict__ perm_in,
                                                         int32_t* __restrict__ perm_out) {
  __shared__ int wsum[16];
  __shared__ int firsts[4];  // actual first two left, first two right positions
  __shared__ uint32_t cmm[2][2];  // children's key min / max (left, right)
  const int h = blockIdx.y, t = threadIdx.x;
  const int4 sg = b.segs[blockIdx.x];
  const int32_t* pi = perm_in + size_t(h) * b.N;
  int32_t* po = perm_out + size_t(h) * b.N;
  if (sg.z == 0) {
    for (int i = t; i < sg.y; i += 1024) po[sg.x + i] = pi[sg.x + i];
    return;
  }
  const size_t si = size_t(h) * b.max_seg + blockIdx.x;
  const uint2 th = b.thr[si];
  const uint32_t* kh = b.keys + size_t(h) * b.N;
  if (PRED && t < 4) {
    firsts[t] = -1;
    cmm[t >> 1][t & 1] = (t & 1) ? 0u : 0xFFFFFFFFu;
  }
  uint32_t mn[2] = {0xFFFFFFFFu, 0xFFFFFFFFu}, mx[2] = {0u, 0u};
  int run_left = 0;
  // four consecutive positions per thread and step (their loads overlap);
  // the scan of the per-thread counts keeps the order stable
  constexpr int PU = 4;
  for (int base = 0; base < sg.y; base += PU * 1024) {
    int lf[PU], cl = 0;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int i = base + PU * t + u;
      lf[u] = (i < sg.y && is_left(kh[sg.x + i], sg.x + i, th)) ? 1 : 0;
      cl += lf[u];
    }
    int tot;
    int lpre = block_excl_scan<int>(cl, wsum, tot) + run_left;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int i = base + PU * t + u;
      const int left = lf[u];
      const int np = left ? sg.x + lpre : sg.x + sg.z + (i - lpre);
      // a left token lands below sg.x + i; a right one stays inside the
      // segment as long as at least sg.z tokens test left, which the exact
      // rank threshold guarantees; the bound keeps a wrong threshold from
      // writing into the next segment or past the head
      if (i < sg.y && np < sg.x + sg.y) {
        const int p = sg.x + i;
        po[np] = pi[p];
        if constexpr (PRED) {
          const size_t hn = size_t(h) * b.N;
          const uint32_t ck = left ? b.keyL[hn + p] : b.keyR[hn + p];
          b.keys_next[hn + np] = ck;
          mn[left ? 0 : 1] = min(mn[left ? 0 : 1], ck);
          mx[left ? 0 : 1] = max(mx[left ? 0 : 1], ck);
          const int rank = left ? lpre : i - lpre;
          if (rank < 2) firsts[(left ? 0 : 2) + rank] = p;
        }
      }
      lpre += lf[u];
    }
    run_left += tot;
  }
  if constexpr (PRED) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      for (int o = 32; o > 0; o >>= 1) {
        mn[c] = min(mn[c], (uint32_t)__shfl_xor((int)mn[c], o, 64));
        mx[c] = max(mx[c], (uint32_t)__shfl_xor((int)mx[c], o, 64));
      }
    if ((t & 63) == 0) {
      atomicMin(&cmm[0][0], mn[0]);
      atomicMax(&cmm[0][1], mx[0]);
      atomicMin(&cmm[1][0], mn[1]);
      atomicMax(&cmm[1][1], mx[1]);
    }
    __syncthreads();
    if (t == 0) {
      const int4 pr = b.pred[si];
      const int kid = b.kids[blockIdx.x];
      const size_t ko = size_t(h) * b.max_seg + kid;
      const bool okl = pr.x >= 0 && pr.x == firsts[0] && pr.y == firsts[1];
      const bool okr = pr.z >= 0 && pr.z == firsts[2] && pr.w == firsts[3];
      b.pred_ok[ko] = okl;
      b.pred_ok[ko + 1] = okr;
      // (min / max of the segments one level down: reset since their last use)
      if (okl) b.segmm[ko] = make_uint2(cmm[0][0], cmm[0][1]);
      if (okr) b.segmm[ko + 1] = make_uint2(cmm[1][0], cmm[1][1]);
    }
  }
  if (b.tot_out) {
    // the final split's side sums are the children's totals (children kid and
    // kid + 1 are adjacent, as the two sides are in ssum)
    const float* ss = b.ssum + si * 2 * b.d;
    float* ct = b.ctot + (size_t(h) * b.max_seg + b.kids[blockIdx.x]) * b.d;
    for (int i = t; i < 2 * b.d; i += 1024) ct[i] = ss[i];
  }
}

// ---------------------------------------------------------------------------
// subtree phase: one workgroup per segment of at most SUB_N tokens
// ---------------------------------------------------------------------------
constexpr int MAXS = 8;        // active segments handled together
constexpr int SUB_LIST = 512;  // active segments per level (leaf >= 4)

__device__ __forceinline__ uint64_t lane_lt() { return (uint64_t(1) << __lane_id()) - 1; }

template <int D>
struct SubShared {
  int pt[SUB_N];          // original token at local position
  int tmp[SUB_N];         // partition target; also select histograms and switcher lists
  uint32_t key[SUB_N];
  uint8_t side[SUB_N];
  uint8_t sid[SUB_N];     // batch slot of the active segment owning a position (255: none)
  float cen[MAXS][2][D];
  float wm[MAXS][2][D];   // per round: c2 - c1, and in [1][0..LPR) each lane slice's share of (c2 - c1).(c1 + c2)
  float ssum[MAXS][2][D];
  float wp[SUB_THREADS / 64][2][D];
  int4 seg[MAXS];         // start, n, n_left
  uint2 thr[MAXS];
  uint32_t spre[MAXS];    // radix select: key digits fixed so far
  int srank[MAXS];        // rank still sought among keys with that prefix
  int scnt[MAXS];         // keys equal to the selected key
  int swc[MAXS];          // tokens that switched side this round
  int done[MAXS];         // split reached a fixed point: later rounds repeat it exactly
  int ndone;
  int2 list[2][SUB_LIST];
  int nlist[2];
};

// For every active segment a of the batch: the rank-n_left (1-based)
// (key, position) pair, i.e. the split threshold.  All threads: four radix
// passes of 8-bit digits with per-segment LDS histograms (aliasing tmp), then
// the position among equal keys (a block sweep when the key is unique, else
// an ordered scan by one wave).
template <int D>
__device__ void subtree_select(SubShared<D>& S, int A, int n0) {
  constexpr int NW = SUB_THREADS / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int(*hist)[256] = reinterpret_cast<int(*)[256]>(S.tmp);
  if (t < A) {
    S.spre[t] = 0u;
    S.srank[t] = S.seg[t].z;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = t; i < A * 256; i += SUB_THREADS) hist[i >> 8][i & 255] = 0;
    __syncthreads();
    for (int i = t; i < n0; i += SUB_THREADS) {
      const int a = S.sid[i];
      if (a == 255 || S.done[a]) continue;
      const uint32_t k = S.key[i];
      if (pass > 0 && (k >> (shift + 8)) != (S.spre[a] >> (shift + 8))) continue;
      atomicAdd(&hist[a][(k >> shift) & 255], 1);
    }
    __syncthreads();
    for (int a = w; a < A; a += NW) {
      if (S.done[a]) continue;
      int c[4], cs = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[a][lane * 4 + j];
        cs += c[j];
      }
      int incl = cs;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int run = incl - cs;
      const int k = S.srank[a];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run < k && k <= run + c[j]) {
          S.spre[a] |= uint32_t(lane * 4 + j) << shift;
          S.srank[a] = k - run;
          if (pass == 3) S.scnt[a] = c[j];
        }
        run += c[j];
      }
    }
    __syncthreads();
  }
  // position of the srank-th equal key (in position order)
  for (int i = t; i < n0; i += SUB_THREADS) {
    const int a = S.sid[i];
    if (a == 255 || S.done[a] || S.scnt[a] != 1) continue;
    if (S.key[i] == S.spre[a]) S.thr[a] = make_uint2(S.spre[a], uint32_t(i));
  }
  for (int a = w; a < A; a += NW) {
    if (S.done[a] || S.scnt[a] == 1) continue;
    const int4 sg = S.seg[a];
    const uint32_t K = S.spre[a];
    const int k = S.srank[a];
    int run = 0;
    for (int base = 0; base < sg.y; base += 64) {
      const int i = base + lane;
      const bool f = i < sg.y && S.key[sg.x + i] == K;
      const uint64_t bal = __ballot(f);
      const int cnt = __popcll(bal);
      if (run + cnt >= k) {
        const uint64_t mine = __ballot(f && int(__popcll(bal & lane_lt())) == k - run - 1);
        if (lane == 0) S.thr[a] = make_uint2(K, uint32_t(sg.x + base + __ffsll((unsigned long long)mine) - 1));
        break;
      }
      run += cnt;
    }
  }
  __syncthreads();
}

// The rows of a root (positions start .. start + n0 - 1, in final order:
// token tok(r) at position start + r) in cluster order, and its leaves'
// means, while the rows are still in the caches.  Roots are whole leaves of
// L positions (the head's last one may be shorter).  Wave w takes leaves w,
// w + NW, ...; lane (row group rsub, slice sub) sums rows rsub, rsub + RPW,
// ... of the leaf, then the row groups are added by a fixed butterfly.
template <typename T, int D, typename Tok>
__device__ void emit_leaves(const T* __restrict__ xh, Tok tok, const LeafOut<T>& lo, int h0, int h, int N,
                            int start, int n0, int L) {
  using G = RowGeo<T, D>;
  constexpr int NW = SUB_THREADS / 64;
  constexpr int U = 4;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int sub = lane % G::LPR, rsub = lane / G::LPR;
  T* xb = h < h0 ? lo.xp0 : lo.xp1;  // null: this tensor's rows are not wanted, only its means
  T* xo = xb ? xb + (size_t(h < h0 ? h : h - h0) * N + start) * D : nullptr;
  float* co = (h < h0 ? lo.c0 + size_t(h) * lo.C * D : lo.c1 + size_t(h - h0) * lo.C * D) +
              size_t(start / L) * D;
  const int nleaf = ceil_div(n0, L);
  for (int f = w; f < nleaf; f += NW) {
    const int r0 = f * L, r1 = min(r0 + L, n0);
    float acc[G::EPV];
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) acc[e] = 0.f;
    for (int rb = r0 + rsub; rb < r1; rb += U * G::RPW) {
      uint4 raw[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int r = rb + q * G::RPW;
        raw[q] = r < r1 ? ld16(xh + size_t(tok(r)) * D + sub * G::EPV) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int r = rb + q * G::RPW;
        if (r < r1) {
          if (xo) *reinterpret_cast<uint4*>(xo + size_t(r) * D + sub * G::EPV) = raw[q];
          float v[G::EPV];
          unpack_vec<T, G::EPV>(raw[q], v);
#pragma unroll
          for (int e = 0; e < G::EPV; ++e) acc[e] += v[e];
        }
      }
    }
#pragma unroll
    for (int o = G::LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < G::EPV; ++e) acc[e] += __shfl_xor(acc[e], o);
    if (rsub == 0) {
      const float inv = 1.f / float(r1 - r0);
#pragma unroll
      for (int e = 0; e < G::EPV; ++e) co[size_t(f) * D + sub * G::EPV + e] = acc[e] * inv;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(SUB_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void subtree_kernel(Src2<T> x, const int32_t* __restrict__ perm,
                                                              int32_t* out0, int32_t* out1,
                                                              const int4* __restrict__ roots, int N,
                                                              int L, int iters, LeafOut<T> lo) {
  using G = RowGeo<T, D>;
  constexpr int NW = SUB_THREADS / 64;
  constexpr int U = 4;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  SubShared<D>& S = *reinterpret_cast<SubShared<D>*>(smem);
  const int h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int4 root = roots[blockIdx.x];
  const int start = root.x, n0 = root.y;
  const int32_t* ph = perm + size_t(h) * N + start;
  int32_t* po = (h < x.h0 ? out0 + size_t(h) * N : out1 + size_t(h - x.h0) * N) + start;
  const T* __restrict__ xh = x.head(h, N, D);
  // a leaf already (possibly longer than SUB_N): its order is final
  if (ceil_div(n0, L) < 2) {
    for (int i = t; i < n0; i += SUB_THREADS) po[i] = ph[i];
    if (lo.c0) emit_leaves<T, D>(xh, [&](int r) { return ph[r]; }, lo, x.h0, h, N, start, n0, L);
    return;
  }
  for (int i = t; i < n0; i += SUB_THREADS) S.pt[i] = ph[i];
  if (t == 0) {
    S.list[0][0] = make_int2(0, n0);
    S.nlist[0] = 1;
  }
  const int sub = lane % G::LPR, rsub = lane / G::LPR;
  int cur = 0;
  __syncthreads();
  while (S.nlist[cur] > 0) {
    const int nl_cur = S.nlist[cur];
    if (t == 0) S.nlist[cur ^ 1] = 0;
    for (int b0 = 0; b0 < nl_cur; b0 += MAXS) {
      const int A = min(MAXS, nl_cur - b0);
      __syncthreads();
      for (int i = t; i < n0; i += SUB_THREADS) S.sid[i] = 255;
      if (t < A) {
        const int2 e = S.list[cur][b0 + t];
        S.seg[t] = make_int4(e.x, e.y, L * ceil_div(ceil_div(e.y, L), 2), 0);
        S.done[t] = 0;
      }
      __syncthreads();
      for (int a = 0; a < A; ++a)
        for (int i = t; i < S.seg[a].y; i += SUB_THREADS) S.sid[S.seg[a].x + i] = uint8_t(a);
      for (int i = t; i < A * 2 * D; i += SUB_THREADS) {
        const int a = i / (2 * D), sdx = (i / D) % 2, col = i % D;
        S.cen[a][sdx][col] = to_f(xh[size_t(S.pt[S.seg[a].x + sdx]) * D + col]);
      }
      // waves per segment for the sums (A <= NW), else one wave loops over segments
      const int wps = A <= NW ? NW / A : 1;
      for (int it = 0; it < iters; ++it) {
        __syncthreads();
        if (t < A) S.swc[t] = 0;
        // the round's per-segment difference of the two means, and each lane
        // slice's share of w . m (m = c1 + c2): delta = 2 (w . x) - w . m
        for (int i = t; i < A * D; i += SUB_THREADS) {
          const int a = i / D, col = i % D;
          S.wm[a][0][col] = S.cen[a][1][col] - S.cen[a][0][col];
        }
        for (int i = t; i < A * G::LPR; i += SUB_THREADS) {
          const int a = i / G::LPR, sb = i % G::LPR;
          float cs = 0.f;
#pragma unroll
          for (int e = 0; e < G::EPV; ++e) {
            const float c1 = S.cen[a][0][sb * G::EPV + e], c2 = S.cen[a][1][sb * G::EPV + e];
            cs = fmaf(c2 - c1, c1 + c2, cs);
          }
          S.wm[a][1][sb] = cs;
        }
        __syncthreads();
        // delta over every position of a segment still moving
        {
          constexpr int STEP = NW * G::RPW;
          // the lane's slice of w and its constant, kept while consecutive
          // rows stay in one segment
          int ca = -1;
          float4 wc[G::EPV / 4];
          float cc = 0.f;
          for (int rb = w * G::RPW; rb < n0; rb += U * STEP) {
            int pp[U], sl[U];
            uint4 raw[U];
#pragma unroll
            for (int q = 0; q < U; ++q) {
              const int r = rb + q * STEP + rsub;
              pp[q] = r < n0 ? r : 0;
              sl[q] = r < n0 ? S.sid[pp[q]] : 255;
              if (sl[q] != 255 && S.done[sl[q]]) sl[q] = 255;
              raw[q] = sl[q] != 255 ? ld16(xh + size_t(S.pt[pp[q]]) * D + sub * G::EPV) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < U; ++q) {
              float v[G::EPV];
              unpack_vec<T, G::EPV>(raw[q], v);
              const int a = sl[q] != 255 ? sl[q] : 0;
              float acc = 0.f;
              if (a != ca) {
                const float4* w4 = reinterpret_cast<const float4*>(&S.wm[a][0][sub * G::EPV]);
#pragma unroll
                for (int e4 = 0; e4 < G::EPV / 4; ++e4) wc[e4] = w4[e4];
                cc = S.wm[a][1][sub];
                ca = a;
              }
#pragma unroll
              for (int e4 = 0; e4 < G::EPV / 4; ++e4) {
                acc = fmaf(wc[e4].x, v[4 * e4], acc);
                acc = fmaf(wc[e4].y, v[4 * e4 + 1], acc);
                acc = fmaf(wc[e4].z, v[4 * e4 + 2], acc);
                acc = fmaf(wc[e4].w, v[4 * e4 + 3], acc);
              }
              acc = fmaf(2.f, acc, -cc);
              acc = row_sum<G::LPR>(acc);
              if (sl[q] != 255 && sub == 0) S.key[pp[q]] = sortable(acc);
            }
          }
        }
        __syncthreads();
        subtree_select<D>(S, A, n0);
        if (it + 1 == iters) break;
        // sums: round 0 both sides, later rounds the tokens that switched side
        for (int a = (A <= NW ? w / wps : w); a < A; a += (A <= NW ? NW : NW)) {
          const int part = A <= NW ? w % wps : 0;
          const int nparts = A <= NW ? wps : 1;
          if (S.done[a]) continue;
          const int4 sg = S.seg[a];
          const uint2 th = S.thr[a];
          int nsw = 0;
          float a0[G::EPV], a1[G::EPV];
#pragma unroll
          for (int e = 0; e < G::EPV; ++e) a0[e] = a1[e] = 0.f;
          if (it == 0) {
            // both sides in full
            const int step = nparts * G::RPW;
            constexpr int U2 = 2;
            for (int rb = part * G::RPW; rb < sg.y; rb += U2 * step) {
              uint4 raw[U2];
              bool lf[U2], ok[U2];
#pragma unroll
              for (int q = 0; q < U2; ++q) {
                const int r = rb + q * step + rsub;
                ok[q] = r < sg.y;
                lf[q] = ok[q] && is_left(S.key[sg.x + r], sg.x + r, th);
                raw[q] = ok[q] ? ld16(xh + size_t(S.pt[sg.x + r]) * D + sub * G::EPV) : make_uint4(0, 0, 0, 0);
              }
#pragma unroll
              for (int q = 0; q < U2; ++q) {
                if (!ok[q]) continue;
                float v[G::EPV];
                unpack_vec<T, G::EPV>(raw[q], v);
                if (lf[q]) {
#pragma unroll
                  for (int e = 0; e < G::EPV; ++e) a0[e] += v[e];
                } else {
#pragma unroll
                  for (int e = 0; e < G::EPV; ++e) a1[e] += v[e];
                }
              }
            }
          } else {
            // only the tokens that switched side: compact their positions (in
            // position order) into this wave's list, then load the rows with
            // every load of a batch in flight
            int* wl = S.tmp + w * 128;
            int nl = 0;
            for (int base = part * 64;; base += nparts * 64) {
              const bool more = base < sg.y;
              if (more) {
                const int r = base + lane;
                const int p = sg.x + r;
                const bool f = r < sg.y && (is_left(S.key[p], p, th) != (S.side[p] != 0));
                const uint64_t bal = __ballot(f);
                if (f) wl[nl + __popcll(bal & lane_lt())] = p;
                nl += __popcll(bal);
              }
              if (nl >= 64 || (!more && nl > 0)) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                constexpr int U3 = 4;
                for (int b = 0; b < nl; b += U3 * G::RPW) {
                  uint4 raw[U3];
                  float sgn[U3];
#pragma unroll
                  for (int q = 0; q < U3; ++q) {
                    const int e = b + q * G::RPW + rsub;
                    sgn[q] = 0.f;
                    raw[q] = make_uint4(0, 0, 0, 0);
                    if (e < nl) {
                      const int pp = wl[e];
                      sgn[q] = is_left(S.key[pp], pp, th) ? 1.f : -1.f;
                      raw[q] = ld16(xh + size_t(S.pt[pp]) * D + sub * G::EPV);
                    }
                  }
#pragma unroll
                  for (int q = 0; q < U3; ++q) {
                    if (sgn[q] == 0.f) continue;
                    float v[G::EPV];
                    unpack_vec<T, G::EPV>(raw[q], v);
                    if (sgn[q] > 0.f) {
#pragma unroll
                      for (int e = 0; e < G::EPV; ++e) a0[e] += v[e];
                    } else {
#pragma unroll
                      for (int e = 0; e < G::EPV; ++e) a0[e] -= v[e];
                    }
                  }
                }
                nsw += nl;
                nl = 0;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
              }
              if (!more) break;
            }
          }
#pragma unroll
          for (int o = G::LPR; o < 64; o <<= 1)
#pragma unroll
            for (int e = 0; e < G::EPV; ++e) {
              a0[e] += __shfl_xor(a0[e], o, 64);
              a1[e] += __shfl_xor(a1[e], o, 64);
            }
          if (lane == 0 && nsw) atomicAdd(&S.swc[a], nsw);
          if (A <= NW) {
            if (rsub == 0)
#pragma unroll
              for (int e = 0; e < G::EPV; ++e) {
                S.wp[w][0][sub * G::EPV + e] = a0[e];
                S.wp[w][1][sub * G::EPV + e] = a1[e];
              }
          } else if (rsub == 0) {
            // this wave alone owns segment a: update its sums and means now
#pragma unroll
            for (int e = 0; e < G::EPV; ++e) {
              const int col = sub * G::EPV + e;
              const float l = it == 0 ? a0[e] : S.ssum[a][0][col] + a0[e];
              const float r = it == 0 ? a1[e] : S.ssum[a][1][col] - a0[e];
              S.ssum[a][0][col] = l;
              S.ssum[a][1][col] = r;
              S.cen[a][0][col] = l / float(sg.z);
              S.cen[a][1][col] = r / float(sg.y - sg.z);
            }
          }
        }
        __syncthreads();
        if (A <= NW) {
          for (int i = t; i < A * 2 * D; i += SUB_THREADS) {
            const int a = i / (2 * D), sdx = (i / D) % 2, col = i % D;
            if (S.done[a]) continue;
            float acc = 0.f;
            for (int j = 0; j < wps; ++j) acc += S.wp[a * wps + j][it == 0 ? sdx : 0][col];
            const float tot = it == 0 ? acc : S.ssum[a][sdx][col] + (sdx == 0 ? acc : -acc);
            S.ssum[a][sdx][col] = tot;
            S.cen[a][sdx][col] = tot / float(sdx == 0 ? S.seg[a].z : S.seg[a].y - S.seg[a].z);
          }
        }
        // sides of this round
        for (int i = t; i < n0; i += SUB_THREADS) {
          const int a = S.sid[i];
          if (a != 255 && !S.done[a]) S.side[i] = is_left(S.key[i], i, S.thr[a]) ? 1 : 0;
        }
        __syncthreads();
        // a round that moved no token fixes the split (and the means) for good
        if (t == 0) {
          int nd = 0;
          for (int a = 0; a < A; ++a) {
            if (it > 0 && !S.done[a] && S.swc[a] == 0) S.done[a] = 1;
            nd += S.done[a];
          }
          S.ndone = nd;
        }
        __syncthreads();
        if (S.ndone == A) break;
      }
      // stable partition of every active segment (one wave each)
      for (int a = w; a < A; a += NW) {
        const int4 sg = S.seg[a];
        const uint2 th = S.thr[a];
        int run_left = 0;
        for (int base = 0; base < sg.y; base += 64) {
          const int i = base + lane;
          const bool valid = i < sg.y;
          const int p = sg.x + i;
          const bool left = valid && is_left(S.key[p], p, th);
          const uint64_t bal = __ballot(left);
          const int pre = __popcll(bal & lane_lt()) + run_left;
          const int np = left ? sg.x + pre : sg.x + sg.z + (i - pre);
          if (valid && np < sg.x + sg.y) S.tmp[np] = S.pt[p];  // bound as in the top phase
          run_left += __popcll(bal);
        }
      }
      __syncthreads();
      for (int a = 0; a < A; ++a)
        for (int i = t; i < S.seg[a].y; i += SUB_THREADS) S.pt[S.seg[a].x + i] = S.tmp[S.seg[a].x + i];
      if (t == 0) {
        int k = S.nlist[cur ^ 1];
        for (int a = 0; a < A; ++a) {
          const int4 sg = S.seg[a];
          if (ceil_div(sg.z, L) >= 2) S.list[cur ^ 1][k++] = make_int2(sg.x, sg.z);
          if (ceil_div(sg.y - sg.z, L) >= 2) S.list[cur ^ 1][k++] = make_int2(sg.x + sg.z, sg.y - sg.z);
        }
        S.nlist[cur ^ 1] = k;
      }
    }
    cur ^= 1;
    __syncthreads();
  }
  __syncthreads();
  for (int i = t; i < n0; i += SUB_THREADS) po[i] = S.pt[i];
  if (lo.c0) emit_leaves<T, D>(xh, [&](int r) { return S.pt[r]; }, lo, x.h0, h, N, start, n0, L);
}

__global__ void leaf_offsets_kernel(int32_t* off0, int32_t* off1, int h0, int C, int N, int L) {
  const int h = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  int32_t* off = h < h0 ? off0 + size_t(h) * (C + 1) : off1 + size_t(h - h0) * (C + 1);
  if (c <= C) off[c] = min(c * L, N);
}

template <typename T, int D>
hipError_t run_bisect(const void* x0, const void* x1, int h0, int H, int N, int L, int iters,
                      const TreePlan& P, int4* segs, int4* chunks, const int32_t* kids, int32_t* pa,
                      int32_t* pb,
                      int32_t* out0, int32_t* out1, void* xp0, void* xp1, float* c0, float* c1, TopBufs b,
                      hipStream_t st) {
  const Src2<T> x{(const T*)x0, (const T*)x1, h0};
  const LeafOut<T> lo{(T*)xp0, (T*)xp1, c0, c1, ceil_div(N, L)};
  const size_t sub_lds = sizeof(SubShared<D>);
  if (hipFuncSetAttribute((const void*)subtree_kernel<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          int(sub_lds)) != hipSuccess)
    return hipErrorInvalidValue;
  int32_t* cur = pa;
  int32_t* nxt = pb;
  bool predicted = false;  // this level's first-round keys were formed by its parent
  // children start from their parent's final side sums (needs a previous
  // round to find the last round's switchers)
  const bool totals = iters >= 2;
  int dir = 0;             // direction of the next full pass over the rows
  for (int lv = 0; lv < P.t.nlev; ++lv) {
    b.segs = segs + P.t.sb[lv];
    b.chunks = chunks + P.t.cb[lv];
    b.kids = kids + P.t.sb[lv];
    b.perm = cur;
    const dim3 gs(P.t.nseg[lv], H), gc(P.t.nchunk[lv], H);
    // predict the children's first round when they stay in the top phase
    const bool predict = iters >= 2 && lv + 1 < P.t.nlev;
    for (int it = 0; it < iters; ++it) {
      const dim3 gd(gc.x * DELTA_SPLIT, gc.y);
      b.rev = dir;
      dir ^= 1;
      if (predict && it + 1 == iters) {
        firsts_kernel<<<gs, 64, 0, st>>>(b);
        delta_kernel<T, D, true><<<gd, 256, 0, st>>>(x, b, 0, 0);
      } else {
        delta_kernel<T, D, false><<<gd, 256, 0, st>>>(x, b, it == 0, it == 0 && predicted);
      }
      b.round = it;
      hist_kernel<<<gc, 256, 0, st>>>(b);
      find_kernel<<<gs, 256, 0, st>>>(b);
      cand_kernel<<<gc, 256, 0, st>>>(b);
      pick_kernel<<<gs, 1024, 0, st>>>(b);
      if (it + 1 < iters) {
        if (it == 0) {
          b.rev = dir;
          dir ^= 1;
          if (lv > 0 && totals) {
            sums_kernel<T, D, true, true><<<gc, 256, 0, st>>>(x, b);
            b.rev = 0;
            update_kernel<D, true, true><<<gs, 256, 0, st>>>(b);
          } else {
            sums_kernel<T, D, true><<<gc, 256, 0, st>>>(x, b);
            b.rev = 0;
            update_kernel<D, true><<<gs, 256, 0, st>>>(b);
          }
        } else {
          b.rev = 0;
          sums_kernel<T, D, false><<<gc, 256, 0, st>>>(x, b);
          update_kernel<D, false><<<gs, 256, 0, st>>>(b);
        }
      } else if (totals && lv + 1 < P.t.nlev) {
        // the final split's side sums (the tokens that switched in the last
        // round), which the partition hands to the children as their totals
        b.rev = 0;
        sums_kernel<T, D, false><<<gc, 256, 0, st>>>(x, b);
        update_kernel<D, false><<<gs, 256, 0, st>>>(b);
      }
    }
    b.tot_out = totals && lv + 1 < P.t.nlev;
    if (predict) {
      partition_kernel<true><<<gs, 1024, 0, st>>>(b, cur, nxt);
      uint32_t* k = b.keys;  // the children's keys become the next level's
      b.keys = b.keys_next;
      b.keys_next = k;
    } else {
      partition_kernel<false><<<gs, 1024, 0, st>>>(b, cur, nxt);
    }
    predicted = predict;
    int32_t* tmp = cur;
    cur = nxt;
    nxt = tmp;
  }
  const int nroots = P.t.nseg[P.t.nlev];
  subtree_kernel<T, D><<<dim3(nroots, H), SUB_THREADS, sub_lds, st>>>(x, cur, out0, out1,
                                                                     segs + P.t.sb[P.t.nlev], N, L, iters, lo);
  return hipGetLastError();
}

}  // namespace

size_t bisect_scratch(int H, int N, int d, int leaf) {
  const TreePlan P = plan_tree(N, leaf, SUB_N);
  Arena a{nullptr, 0, 0};
  a.get<int4>(size_t(P.total_seg));
  a.get<int4>(size_t(P.total_chunk + 1));
  a.get<int32_t>(size_t(H) * N);   // perm ping-pong
  a.get<int32_t>(size_t(H) * N);
  a.get<uint32_t>(size_t(H) * N);  // keys
  a.get<uint8_t>(size_t(H) * N);   // side
  a.get<float>(size_t(H) * P.max_seg * 2 * d);   // cen
  a.get<float>(size_t(H) * P.max_seg * 2 * d);   // ssum
  a.get<uint2>(size_t(H) * P.max_seg);
  a.get<float>(size_t(H) * P.max_chunk * 2 * d);
  a.get<uint2>(size_t(H) * P.max_seg);
  a.get<int32_t>(size_t(H) * P.max_seg * NBIN);
  a.get<int2>(size_t(H) * P.max_seg);
  a.get<unsigned long long>(size_t(H) * P.max_seg * CAND_CAP);
  a.get<int32_t>(size_t(H) * P.max_seg);
  a.get<int32_t>(size_t(P.total_seg));  // kids
  a.get<int4>(size_t(H) * P.max_seg);   // pred
  a.get<uint32_t>(size_t(H) * N);       // keyL
  a.get<uint32_t>(size_t(H) * N);       // keyR
  a.get<uint32_t>(size_t(H) * N);       // keys_next
  a.get<int32_t>(size_t(H) * P.max_seg);  // pred_ok
  a.get<float>(size_t(H) * P.max_seg * d);  // ctot
  return a.used;
}

hipError_t bisect_run(const void* x0, const void* x1, int h0, int dtype, int H, int N, int d, int leaf,
                      int iters, int32_t* perm0, int32_t* perm1, int32_t* off0, int32_t* off1, void* xp0,
                      void* xp1, float* cen0, float* cen1, Arena& s, hipStream_t st) {
  const TreePlan P = plan_tree(N, leaf, SUB_N);
  int4* segs = s.get<int4>(size_t(P.total_seg));
  int4* chunks = s.get<int4>(size_t(P.total_chunk + 1));
  int32_t* pa = s.get<int32_t>(size_t(H) * N);
  int32_t* pb = s.get<int32_t>(size_t(H) * N);
  TopBufs b{};
  b.keys = s.get<uint32_t>(size_t(H) * N);
  b.side = s.get<uint8_t>(size_t(H) * N);
  b.cen = s.get<float>(size_t(H) * P.max_seg * 2 * d);
  b.ssum = s.get<float>(size_t(H) * P.max_seg * 2 * d);
  b.thr = s.get<uint2>(size_t(H) * P.max_seg);
  b.part = s.get<float>(size_t(H) * P.max_chunk * 2 * d);
  b.segmm = s.get<uint2>(size_t(H) * P.max_seg);
  b.ghist = s.get<int32_t>(size_t(H) * P.max_seg * NBIN);
  b.selbin = s.get<int2>(size_t(H) * P.max_seg);
  b.cand = s.get<unsigned long long>(size_t(H) * P.max_seg * CAND_CAP);
  b.ccount = s.get<int32_t>(size_t(H) * P.max_seg);
  int32_t* kids = s.get<int32_t>(size_t(P.total_seg));
  b.pred = s.get<int4>(size_t(H) * P.max_seg);
  b.keyL = s.get<uint32_t>(size_t(H) * N);
  b.keyR = s.get<uint32_t>(size_t(H) * N);
  b.keys_next = s.get<uint32_t>(size_t(H) * N);
  b.pred_ok = s.get<int32_t>(size_t(H) * P.max_seg);
  b.ctot = s.get<float>(size_t(H) * P.max_seg * d);
  b.d = d;
  b.max_seg = P.max_seg;
  b.max_chunk = P.max_chunk;
  b.N = N;
  // the top levels ping-pong between two scratch orders; the subtree phase
  // writes each head's final order to its tensor's output
  iota_kernel<<<dim3(ceil_div(N, 256), H), 256, 0, st>>>(pa, N);
  const size_t ncnt = size_t(H) * P.max_seg;
  zero_i32<<<unsigned((ncnt + 255) / 256), 256, 0, st>>>(b.ccount, ncnt);
  zero_i32<<<unsigned((ncnt * NBIN + 255) / 256), 256, 0, st>>>(b.ghist, ncnt * NBIN);
  init_minmax<<<unsigned((ncnt + 255) / 256), 256, 0, st>>>(b.segmm, ncnt);
  build_tree_kernel<<<1, 1024, 0, st>>>(P.t, N, segs, chunks, kids);
  hipError_t e;
  if (dtype == SA_F32 && d == 64)
    e = run_bisect<float, 64>(x0, x1, h0, H, N, leaf, iters, P, segs, chunks, kids, pa, pb, perm0, perm1, xp0, xp1,
                                   cen0, cen1, b, st);
  else if (dtype == SA_F32 && d == 128)
    e = run_bisect<float, 128>(x0, x1, h0, H, N, leaf, iters, P, segs, chunks, kids, pa, pb, perm0, perm1, xp0, xp1,
                                   cen0, cen1, b, st);
  else if (dtype == SA_BF16 && d == 64)
    e = run_bisect<bf16_t, 64>(x0, x1, h0, H, N, leaf, iters, P, segs, chunks, kids, pa, pb, perm0, perm1, xp0, xp1,
                                   cen0, cen1, b, st);
  else
    e = run_bisect<bf16_t, 128>(x0, x1, h0, H, N, leaf, iters, P, segs, chunks, kids, pa, pb, perm0, perm1, xp0, xp1,
                                   cen0, cen1, b, st);
  if (e != hipSuccess) return e;
  const int C = ceil_div(N, leaf);
  leaf_offsets_kernel<<<dim3(ceil_div(C + 1, 256), H), 256, 0, st>>>(off0, off1, h0, C, N, leaf);
  return hipGetLastError();
}

}  // namespace sa
