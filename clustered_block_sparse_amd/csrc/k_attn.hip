// Block-sparse attention over the selected key clusters, with optional mean
// compensation of the excluded ones, writing rows back in original order.
//
// SCOPE (English abstract): attention runs over the selected original keys
// and values.  ClusterAttention (English abstract): clusters are contiguous
// power-of-two blocks so block-sparse attention keeps dense per-pair
// throughput, and an excluded cluster is compensated through its mean.  The
// closed form for a query n of query cluster i (sel = keys of the selected
// key clusters, excl = the non-empty excluded clusters, c = compensation):
//   O_n = [sum_sel e^{s_nm} v_m + c sum_excl |K_j| e^{<q_n,kbar_j>s} vbar_j]
//       / [sum_sel e^{s_nm}     + c sum_excl |K_j| e^{<q_n,kbar_j>s}]
//
// Layout.  Keys/values are in key-cluster order, so a query cluster's
// selection is a short list of contiguous row ranges (adjacent selected
// clusters merged).  A workgroup owns one tile of up to 128 query rows of one
// query cluster and streams the concatenated ranges in 64-key tiles; the
// compensation runs afterwards over "pseudo keys" (one per key cluster) whose
// logit carries the bias ln|K_j| (-inf where selected or empty).
//
// Rows whose ranges all start at multiples of 64 (and end at one or at N)
// stream whole 64-key blocks of K and V rows by direct buffer-to-LDS loads.
// Other rows (and SCOPE's key combos) gather their key rows one by one:
// before each tile one wave lists the key row of each position, and the K and
// V rows then arrive by direct buffer-to-LDS loads too, each lane's source
// offset taken from the listed row of the slot it fills.
//
// bf16 path: 4 waves x 32 query rows.  S^T = K Q^T on 32x32x16 bf16 MFMA so
// every lane owns one query column and keeps the online-softmax state in
// registers; P stays in registers and feeds O^T = V^T P^T directly, whose V^T
// operand comes from row-major V tiles by the LDS transpose read.  Rescaling
// is lazy (only when the running max grows by more than 2^8).  The cluster
// means enter the compensation as bf16 rows, 64 clusters to a tile, through
// the same pipeline.
// fp32 path: one thread per query row, fp32 FMA (parity-grade, small inputs).

#include <math.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;      // keys per tile
constexpr int HK = 32;      // keys per half tile (one 32x32 MFMA block)
constexpr int TQ = 128;     // query rows per workgroup (upper bound)
constexpr int RCH = 512;    // ranges staged in LDS at a time
constexpr int ALIGNED_MAX_CK = 4096;  // key clusters up to which rows get precomputed ranges
constexpr float LOG2E = 1.4426950408889634f;
// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format)
constexpr int BUF_DWORD3 = 0x00020000;

struct Prep {
  int4* tiles;        // [H][maxT] {cluster, first position, rows, 0}
  int32_t* ntiles;    // [H]
  int2* ranges;       // [H][Cq][Rmax] {start, end}
  int32_t* rcount;    // [H][Cq]
  int32_t* raligned;  // [H][Cq] 1 if every range starts at a multiple of 64 and ends at one or at N
  int32_t* korder;    // [H][Ck] key clusters by how many query clusters selected them (most first)
  int2* krange;       // [H][Ck] key positions {start, end} of those clusters, in the same order
  bf16_t* kbh;        // [H][Ckp][D]  kbar, bf16
  bf16_t* vbr;        // [H][Ckp][D]  vbar, bf16
  float* logsz;       // [H][Ckp]  ln|K_j| or -inf for empty
  float* kbf;         // fp32 path: [H][Ckp][D]
  float* vbf;         // fp32 path: [H][Ckp][D]
  int maxT, Rmax, Ckp, W;
};

// --------------------------------------------------------------------------
// preparation
// --------------------------------------------------------------------------
// Walk order of a head's key clusters: by the number of query clusters that
// selected each (most first, ties by index).  Tiles that run side by side on
// one XCD then reach their shared key blocks at about the same step, while the
// XCD's L2 still holds them (in ascending order the positions of a shared
// cluster drift apart by the clusters only one of the rows selected).  One
// workgroup per head: selection counts in LDS, each cluster's rank by
// counting the clusters ahead of it.
constexpr int RANK_THREADS = 1024;
__global__ __launch_bounds__(RANK_THREADS) void key_rank_kernel(const uint32_t* __restrict__ mask,
                                                                const int32_t* __restrict__ k_off, int Cq, int Ck,
                                                                int W, int32_t* __restrict__ korder,
                                                                int2* __restrict__ krange) {
  __shared__ int pop[ALIGNED_MAX_CK];
  const int h = blockIdx.x, t = threadIdx.x;
  const uint32_t* mh = mask + size_t(h) * Cq * W;
  for (int j = t; j < Ck; j += RANK_THREADS) pop[j] = 0;
  __syncthreads();
  // coalesced mask words; each set bit adds one to its cluster (integer LDS
  // atomics: the counts do not depend on their order)
  for (int e = t; e < Cq * W; e += RANK_THREADS) {
    const int wc = e % W;
    uint32_t m = mh[e];
    if (wc == W - 1 && (Ck & 31)) m &= (1u << (Ck & 31)) - 1u;
    while (m) {
      atomicAdd(&pop[wc * 32 + __ffs(m) - 1], 1);
      m &= m - 1u;
    }
  }
  __syncthreads();
  for (int j = t; j < Ck; j += RANK_THREADS) {
    const int pj = pop[j];
    int r = 0;
    for (int i = 0; i < Ck; ++i) {
      const int pi = pop[i];
      r += (pi > pj || (pi == pj && i < j)) ? 1 : 0;
    }
    korder[size_t(h) * Ck + r] = j;
    krange[size_t(h) * Ck + r] = make_int2(k_off[size_t(h) * (Ck + 1) + j], k_off[size_t(h) * (Ck + 1) + j + 1]);
  }
}

// Row i's selected key clusters as ranges of key positions, in the head's
// walk order (one range per non-empty cluster) when the row selects at most
// Rmax clusters; otherwise in ascending order with adjacent clusters merged
// (at most Ck/2 + 1 ranges).  Either way a range ending at N (the only one
// whose last tile can be partial) comes last.
__global__ __launch_bounds__(64) void ranges_kernel(const uint32_t* __restrict__ mask,
                                                    const int32_t* __restrict__ k_off, int Cq,
                                                    int Ck, int W, int Rmax, int N,
                                                    const int32_t* __restrict__ korder,
                                                    const int2* __restrict__ krange,
                                                    int2* __restrict__ ranges,
                                                    int32_t* __restrict__ rcount,
                                                    int32_t* __restrict__ raligned) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const uint32_t* mr = mask + (size_t(h) * Cq + i) * W;
  const int32_t* ko = k_off + size_t(h) * (Ck + 1);
  int2* out = ranges + (size_t(h) * Cq + i) * Rmax;
  bool misaligned = false;
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  // the row's mask words in registers (word w in lane w % 64 of register
  // w / 64; Ck <= 4096, so at most two)
  uint32_t mw0 = 0, mw1 = 0;
  if (lane < W) mw0 = mr[lane];
  if (lane + 64 < W) mw1 = mr[lane + 64];
  const uint32_t tail = (Ck & 31) ? (1u << (Ck & 31)) - 1u : ~0u;
  if (lane == W - 1) mw0 &= tail;
  if (lane + 64 == W - 1) mw1 &= tail;
  int nsel = __popc(mw0) + __popc(mw1);
  for (int o = 32; o > 0; o >>= 1) nsel += __shfl_xor(nsel, o);
  int ns = 0;
  if (nsel <= Rmax && Ck <= 4096) {
    const int32_t* ord = korder + size_t(h) * Ck;
    const int2* kr = krange + size_t(h) * Ck;
    int last_a = -1;  // start of the selected cluster ending at N
    for (int r0 = 0; r0 < Ck; r0 += 64) {
      const int r = r0 + lane;
      int j = 0;
      int2 ab = make_int2(0, 0);
      if (r < Ck) {
        j = ord[r];
        ab = kr[r];
      }
      const int wd = j >> 5;
      const uint32_t w0 = __shfl(mw0, wd & 63), w1 = __shfl(mw1, wd & 63);  // every lane takes part
      const uint32_t word = wd < 64 ? w0 : w1;
      const int a = ab.x, b = ab.y;
      const bool sel = r < Ck && ((word >> (j & 31)) & 1u);
      const bool at_end = sel && b > a && b == N;
      const bool take = sel && b > a && !at_end;
      const uint64_t bt = __ballot(take), bl = __ballot(at_end);
      if (take) {
        out[ns + __popcll(bt & lt)] = make_int2(a, b);
        misaligned |= (a & (KT - 1)) != 0 || (b & (KT - 1)) != 0;
      }
      ns += __popcll(bt);
      if (bl) last_a = __shfl(a, __ffsll((unsigned long long)bl) - 1);
    }
    if (last_a >= 0) {
      if (lane == 0) out[ns] = make_int2(last_a, N);
      misaligned |= lane == 0 && (last_a & (KT - 1)) != 0;
      ++ns;
    }
  } else {
    int ne = 0;
    for (int j0 = 0; j0 < Ck; j0 += 64) {
      const int j = j0 + lane;
      const bool in = j < Ck;
      const bool sel = in && ((mr[j >> 5] >> (j & 31)) & 1u);
      const bool selp = in && j > 0 && ((mr[(j - 1) >> 5] >> ((j - 1) & 31)) & 1u);
      const bool seln = in && (j + 1 < Ck) && ((mr[(j + 1) >> 5] >> ((j + 1) & 31)) & 1u);
      const bool st = sel && !selp;
      const bool en = sel && !seln;
      const uint64_t bs = __ballot(st), be = __ballot(en);
      if (st) {
        out[ns + __popcll(bs & lt)].x = ko[j];
        misaligned |= (ko[j] & (KT - 1)) != 0;
      }
      if (en) {
        out[ne + __popcll(be & lt)].y = ko[j + 1];
        misaligned |= (ko[j + 1] & (KT - 1)) != 0 && ko[j + 1] != N;
      }
      ns += __popcll(bs);
      ne += __popcll(be);
    }
  }
  const bool any_mis = __ballot(misaligned) != 0;
  if (lane == 0) {
    rcount[size_t(h) * Cq + i] = ns;
    raligned[size_t(h) * Cq + i] = any_mis ? 0 : 1;
  }
}

__global__ void fill_zero_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ q_off, int Cq,
                                                     int rows, int maxT, int4* __restrict__ tiles,
                                                     int32_t* __restrict__ ntiles) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int h = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int32_t* qo = q_off + size_t(h) * (Cq + 1);
  if (t == 0) carry = 0;
  __syncthreads();
  for (int b = 0; b < Cq; b += 1024) {
    const int i = b + t;
    const int sz = i < Cq ? qo[i + 1] - qo[i] : 0;
    const int nt = ceil_div(sz, rows);
    int x = nt;
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int pre = carry;
    for (int j = 0; j < w; ++j) pre += wsum[j];
    pre += x - nt;
    for (int u = 0; u < nt; ++u)
      if (pre + u < maxT)
        tiles[size_t(h) * maxT + pre + u] = make_int4(i, qo[i] + u * rows, min(rows, sz - u * rows), 0);
    __syncthreads();
    if (t == 1023) carry = pre + nt;
    __syncthreads();
  }
  if (t == 0) ntiles[h] = carry;
}

// ---------------------------------------------------------------------------
// LDS tile layout of the MFMA kernel.  Tiles are unpadded; bank conflicts are
// avoided by XOR-swizzling the 16-byte chunks of a row, so whole tiles can
// arrive by direct global->LDS loads (lane l of such a load lands at 16 l).
//   K tile: KT rows of D bf16; chunk c of row r at chunk c ^ swz(r).
//   V tile: two half tiles (keys 0..31 and 32..63) of 32 rows of D bf16;
//           chunk c of row r at chunk c ^ vswz(r) (below).
// swz puts the chunks any 16 consecutive rows (or any 8) read at one column on
// distinct banks, for 64 as for 32 LDS banks.
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) return r & 15;
  else return (r & 7) ^ ((r >> 3) & 1);  // CPR == 8
}
// element offset of 16-byte chunk c of row r in a tile of CPR chunks per row
template <int CPR>
__device__ __forceinline__ int toff(int r, int c) {
  return r * (CPR * 8) + ((c ^ swz<CPR>(r)) << 3);
}

// V half tiles are row-major too (32 keys of D columns) and are read with the
// LDS transpose read: within each 16-lane group, lane i receives element i % 4
// of the 8-byte pieces addressed by lanes i / 4 + 4 j (j = 0..3).  Lanes that
// address 4 keys x 4 column pieces thus receive 4 keys of one column each,
// which is the A operand of O^T = V^T P^T, so V needs no transposed copy.
// Their chunks are XOR-swizzled by 2 (r mod CPR/2): every 16-lane group of such
// a read then meets 32 distinct banks, and a wave each of 64 banks twice (the
// best XOR swizzle of the row bits, found by exhaustive search).
template <int CPR>
__device__ __forceinline__ int vswz(int r) {
  return (r & (CPR / 2 - 1)) << 1;
}
template <int CPR>
__device__ __forceinline__ int vtoff(int r, int c) {
  return r * (CPR * 8) + ((c ^ vswz<CPR>(r)) << 3);
}
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_t __attribute__((address_space(3)))*)p);
  return __builtin_bit_cast(uint2, r);
}

__global__ __launch_bounds__(128) void comp_prep_kernel(const float* __restrict__ kbar,
                                                        const float* __restrict__ vbar,
                                                        const int32_t* __restrict__ k_off, int Ck,
                                                        int Ckp, int D, bf16_t* kbh,
                                                        bf16_t* vbr, float* kbf, float* vbf,
                                                        float* logsz) {
  const int j = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const size_t o = (size_t(h) * Ckp + j) * D;
  const bool in = j < Ck;
  int sz = 0;
  if (in) sz = k_off[size_t(h) * (Ck + 1) + j + 1] - k_off[size_t(h) * (Ck + 1) + j];
  for (int c = t; c < D; c += 128) {
    const float kv = (in && sz > 0) ? kbar[(size_t(h) * Ck + j) * D + c] : 0.f;
    const float vv = (in && sz > 0) ? vbar[(size_t(h) * Ck + j) * D + c] : 0.f;
    if (kbh) {
      kbh[o + c] = f2bf(kv);
      vbr[o + c] = f2bf(vv);
    }
    if (kbf) {
      kbf[o + c] = kv;
      vbf[o + c] = vv;
    }
  }
  if (t == 0) logsz[size_t(h) * Ckp + j] = sz > 0 ? logf(float(sz)) : -__builtin_huge_valf();
}

// Workgroup -> (head, tile).  Workgroups go to the 8 XCDs round-robin by
// linear id, and each XCD starts them in id order.  XCD x takes, head after
// head, the x-th eighth of that head's tiles: every XCD works on a contiguous
// run of neighbouring query clusters (whose key blocks its own L2 can share),
// while all XCDs stay on the same one or two heads at a time, whose K and V
// fit the memory-side cache together.  Each head owns ceil(maxT / 8) slots
// per XCD, of which the first ceil(ntiles / 8) carry tiles, so padding (maxT
// is only an upper bound) is spread evenly over the XCDs.  The grid is
// 8 * H * ceil(maxT / 8); h = H or tix = -1 marks a padding workgroup.
__device__ __forceinline__ void map_tile(int maxT, int H, const int32_t* ntiles, int& h, int& tix) {
  const int t8 = (maxT + 7) / 8;
  const int b = blockIdx.x, x = b & 7, k = b >> 3;
  h = k / t8;
  tix = -1;
  if (h >= H) return;
  const int nt = ntiles[h], n8 = (nt + 7) / 8, kk = k % t8;
  if (kk < n8 && x * n8 + kk < nt) tix = x * n8 + kk;
}

// Stage the next selected key clusters of a row, in cluster order, straight
// from its mask bits: rs[k] = first key position of the k-th staged cluster,
// rp[k] = keys staged before it (rp[n] = total).  Wave 0 scans 16 mask words
// (512 clusters) at a time while they fit in RCH entries; `word` is the scan
// position, shared through sh[0].  Returns the number of clusters staged (0:
// the row is exhausted).  Called by the whole block.
__device__ int fill_chunk(const uint32_t* __restrict__ mr, int W, int Ck, const int32_t* __restrict__ ko,
                          int* rs, int* rp, int* wsum, int* sh) {
  const int t = threadIdx.x, lane = t & 63;
  if (t < 64) {
    int word = sh[0];
    int nr = 0;
    while (word < W) {
      uint32_t bits = 0;
      const int wi = word + lane;
      if (lane < 16 && wi < W) {
        bits = mr[wi];
        const int rem = Ck - 32 * wi;
        if (rem < 32) bits &= (1u << rem) - 1u;
      }
      int c = __popc(bits);
      int x = c;
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const int blk = __shfl(x, 63, 64);
      if (nr + blk > RCH) break;
      int slot = nr + x - c;
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        const int j = 32 * wi + b;
        rs[slot] = ko[j];
        rp[slot] = ko[j + 1] - ko[j];
        ++slot;
      }
      nr += blk;
      word += 16;
    }
    if (lane == 0) {
      sh[0] = word;
      sh[1] = nr;
    }
  }
  __syncthreads();
  const int nrc = sh[1];
  // lengths -> exclusive prefix (block scan over nrc entries)
  const int lane2 = t & 63, w = t >> 6, nw = blockDim.x >> 6;
  int carry = 0;
  for (int b = 0; b < nrc; b += blockDim.x) {
    const int k = b + t;
    const int len = k < nrc ? rp[k] : 0;
    int x = len;
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane2 >= o) x += y;
    }
    if (lane2 == 63) wsum[w] = x;
    __syncthreads();
    int pre = carry, tot = 0;
    for (int j = 0; j < nw; ++j) {
      if (j < w) pre += wsum[j];
      tot += wsum[j];
    }
    if (k < nrc) rp[k] = pre + x - len;
    carry += tot;
    __syncthreads();
  }
  if (t == 0) rp[nrc] = carry;
  __syncthreads();
  return nrc;
}

// --------------------------------------------------------------------------
// fp32 (and generic) path: one thread per query row
// --------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_simple(AttnArgs a, Prep p, float scale) {
  __shared__ float Ks[32][D];
  __shared__ float Vs[32][D];
  __shared__ int rs[RCH + 1], rp[RCH + 1];
  __shared__ int wsum[16];
  __shared__ int fsh[2];
  __shared__ float bias[32];
  int h, tix;
  map_tile(p.maxT, a.H, p.ntiles, h, tix);
  if (h >= a.H || tix < 0) return;
  const int4 td = p.tiles[size_t(h) * p.maxT + tix];
  const int i = td.x, p0 = td.y, nr = td.z;
  const int t = threadIdx.x;
  const int N = a.N;
  const bool qv = t < nr;
  const T* qp = a.q_src ? (const T*)a.q_src + (size_t(h) * N + a.q_idx[size_t(h) * N + p0 + (qv ? t : 0)]) * D
                        : (const T*)a.q_perm + (size_t(h) * N + p0 + (qv ? t : 0)) * D;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = to_f(qp[c]) * scale;
    o[c] = 0.f;
  }
  float m = -__builtin_huge_valf(), l = 0.f;
  const T* kh = (const T*)a.k_perm + size_t(h) * N * D;
  const T* vh = (const T*)a.v_perm + size_t(h) * N * D;
  const uint32_t* mrow = a.mask + (size_t(h) * a.Cq + i) * p.W;
  const int32_t* kof = a.k_off + size_t(h) * (a.Ck + 1);
  auto consume = [&](int nk, const float* bs) {
    for (int kk = 0; kk < nk; ++kk) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(q[c], Ks[kk][c], s);
      if (bs) s += bs[kk];
      if (s == -__builtin_huge_valf()) continue;
      if (s > m) {
        const float al = expf(m - s);
        l *= al;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= al;
        m = s;
      }
      const float pr = expf(s - m);
      l += pr;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(pr, Vs[kk][c], o[c]);
    }
  };
  int scan_word = 0;  // mask scan position
  while (true) {
    __syncthreads();
    if (t == 0) fsh[0] = scan_word;
    __syncthreads();
    const int nrc = fill_chunk(mrow, p.W, a.Ck, kof, rs, rp, wsum, fsh);
    scan_word = fsh[0];
    if (nrc == 0) break;
    const int total = rp[nrc];
    for (int base = 0; base < total; base += 32) {
      const int nk = min(32, total - base);
      __syncthreads();
      for (int v = t; v < 32 * D; v += 128) {
        const int kk = v / D, c = v % D;
        float kv = 0.f, vv = 0.f;
        if (kk < nk) {
          // binary search the cluster of position base+kk
          const int pos = base + kk;
          int lo = 0, hi = nrc - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rp[mid] <= pos) lo = mid; else hi = mid - 1;
          }
          const int row = rs[lo] + (pos - rp[lo]);
          kv = to_f(kh[size_t(row) * D + c]);
          vv = to_f(vh[size_t(row) * D + c]);
        }
        Ks[kk][c] = kv;
        Vs[kk][c] = vv;
      }
      __syncthreads();
      consume(nk, nullptr);
    }
  }
  if (a.compensate) {
    const uint32_t* mr = a.mask + (size_t(h) * a.Cq + i) * p.W;
    for (int j0 = 0; j0 < a.Ck; j0 += 32) {
      const int nk = min(32, a.Ck - j0);
      __syncthreads();
      for (int v = t; v < 32 * D; v += 128) {
        const int kk = v / D, c = v % D;
        const size_t src = (size_t(h) * p.Ckp + j0 + kk) * D + c;
        Ks[kk][c] = kk < nk ? p.kbf[src] : 0.f;
        Vs[kk][c] = kk < nk ? p.vbf[src] : 0.f;
      }
      if (t < 32) {
        const int j = j0 + t;
        float b = -__builtin_huge_valf();
        if (t < nk && !((mr[j >> 5] >> (j & 31)) & 1u)) b = p.logsz[size_t(h) * p.Ckp + j];
        bias[t] = b;
      }
      __syncthreads();
      consume(nk, bias);
    }
  }
  if (qv) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int32_t orig = a.q_idx[size_t(h) * N + p0 + t];
    T* op = (T*)a.o + (size_t(h) * N + orig) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = from_f<T>(o[c] * inv);
    if (a.lse) a.lse[size_t(h) * N + orig] = l > 0.f ? m + logf(l) : -__builtin_huge_valf();
  }
}

// --------------------------------------------------------------------------
// bf16 MFMA path
// --------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx16 mfma32(bf16x8_t a, bf16x8_t b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// 16 bytes per lane from a raw buffer over [base, base + nbytes) into LDS
// (lane l of the wave lands at lds + 16 l); `off` is the lane's byte offset.
// The record count is unsigned 32-bit: nbytes carries sizes up to 2^32 - 1
// (callers form it in uint32_t arithmetic; a head's rows stay below 4 GiB).
__device__ __forceinline__ void buf_load_lds16(const void* base, int nbytes, bf16_t* lds, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nbytes, BUF_DWORD3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, 0);
}

// max and sum of a value over lanes l and l ^ 32.  v_permlane32_swap trades
// the upper half of one copy with the lower half of the other (no LDS round
// trip), so every lane finds both values among the two results.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, uint32_t(r[0])), __builtin_bit_cast(float, uint32_t(r[1])));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, uint32_t(r[0])) + __builtin_bit_cast(float, uint32_t(r[1]));
}

// p[i] of memory that no thread writes during the kernel, read through the
// constant address space (a scalar load when the index is uniform, so the
// vector-memory counter is left to the tile loads)
__device__ __forceinline__ int2 const_load_int2(const int2* p, int i) {
  const __attribute__((address_space(4))) long long* q = (const __attribute__((address_space(4))) long long*)p;
  const long long v = q[i];
  return make_int2(int(v), int(v >> 32));
}

#define BF16_ONES (__builtin_bit_cast(bf16x2_t, 0x3F803F80u))  // (1.0, 1.0)

// two floats -> packed bf16 pair (hardware round-to-nearest-even)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
struct MfmaLds {
  int rs[RCH + 1];
  int rp[RCH + 1];
  int wsum[16];
  int fsh[2];
  int rowidx[3][KT];  // general path: key row of each position of tile t in [t % 3]
  float cbias[3][KT];  // compensation: score bias of the n-th live tile of cluster means in [n % 3]
};

// ALIGNED: rows whose ranges are 64-aligned stream whole 64-key blocks (K and
// V rows are plain 16-byte copies); the other instantiation gathers rows of
// arbitrary ranges, each lane's direct load taking its listed key row.  Each
// workgroup runs in the instantiation matching its row and exits in the other.
template <int D, bool ALIGNED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && ALIGNED ? 3 : 2, D == 64 && ALIGNED ? 3 : 2))) void attn_mfma(AttnArgs a, Prep p, float sl2) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int DS = D / 16;         // MFMA k-steps over d
  constexpr int DT = D / 32;         // 32-row tiles of d in O^T
  constexpr int DG = D / 8;          // 16-byte chunks of a K / Q / O row
  constexpr int CK = KT * D / 8 / 256;  // 16-byte chunks per thread of a K tile
  constexpr int CH = CK / 2;            // ... of a V half tile
  // Six separate tiles: K double buffered, and V split into its lower and
  // upper 32 keys (VL, VH), each double buffered.  As distinct objects, a
  // direct load into one is visibly independent of reads from the others.
  __shared__ __attribute__((aligned(16))) bf16_t K0[KT * D], K1[KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t VL0[D * HK], VL1[D * HK], VH0[D * HK], VH1[D * HK];
  __shared__ __attribute__((aligned(16))) MfmaLds<D> S;

  int h, tix;
  map_tile(p.maxT, a.H, p.ntiles, h, tix);
  if (h >= a.H || tix < 0) return;
  const int4 td = p.tiles[size_t(h) * p.maxT + tix];
  const int i = td.x, p0 = td.y, nr = td.z;
  if ((p.raligned[size_t(h) * a.Cq + i] != 0) != ALIGNED) return;
  // the wave index is uniform across the wave: keep it (and what derives from it) in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hi = lane >> 5;
  const int N = a.N;

  // Q fragments (B operand of S^T = K Q^T): query 32w+col, d = 16s + 8hi + e
  const int qr = 32 * w + col;
  const bool qv = qr < nr;
  // query rows from the cluster-order copy, or from the original order
  // through the cluster permutation
  const bf16_t* qrow =
      a.q_src ? (const bf16_t*)a.q_src + (size_t(h) * N + a.q_idx[size_t(h) * N + p0 + (qv ? qr : 0)]) * D
              : (const bf16_t*)a.q_perm + (size_t(h) * N + p0 + (qv ? qr : 0)) * D;
  bf16x8_t qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 u = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hi);
    if (!qv) u = make_uint4(0, 0, 0, 0);
    qf[s] = as_bf8(u);
  }

  floatx16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m = -__builtin_huge_valf();  // running max, log2 domain
  float lsum = 0.f;                   // this lane's share of the denominator

  const bf16_t* kh = (const bf16_t*)a.k_perm + size_t(h) * N * D;

  // Score tiles are handled in 32-key halves: half kt of a 64-key tile is one
  // 32x32 block of S^T, whose lane (col, hi) holds keys
  // 32 kt + 8 (r / 4) + 4 hi + r % 4 (r = 0..15) of query column col.
  auto zero16 = [&](floatx16& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
  };
  // S^T half kt = K[32 kt .. 32 kt + 31] Q^T; all K fragments are read first,
  // so LDS latency is paid once per half
  auto qk_half = [&](floatx16& s, const bf16_t* Kb, int kt) {
    uint4 kf[DS];
#pragma unroll
    for (int st = 0; st < DS; ++st)
      kf[st] = *reinterpret_cast<const uint4*>(Kb + toff<DG>(32 * kt + col, 2 * st + hi));
#pragma unroll
    for (int st = 0; st < DS; ++st) s = mfma32(as_bf8(kf[st]), qf[st], s);
  };
  // keys of half kt at or past nvalid -> -inf (the constant part of the key
  // index is compared with nvalid - 32 kt - 4 hi)
  auto mask_half = [&](floatx16& s, int nvalid, int kt) {
    const int lim = nvalid - 32 * kt - 4 * hi;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -__builtin_huge_valf();
  };
  // log2-domain maximum of a half's scores over the query column
  auto max_half = [&](const floatx16& s, float lsc) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    return pair_max(mx) * lsc;
  };
  // lazy rescale: the running maximum moves only when a block's maximum
  // exceeds it by more than 2^8, so probabilities stay below 256
  auto rescale_to = [&](float mx) {
    float alpha = 1.f;
    if (mx > m + 8.f) {
      alpha = __builtin_amdgcn_exp2f(m - mx);  // m = -inf -> 0
      m = mx;
    }
    if (__ballot(alpha != 1.f)) {
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
  };
  // P = 2^(s lsc - m) as packed bf16 pairs, the B operand of P V; the row sum
  // adds the same bf16 values (dot2 against (1, 1))
  auto exp_half = [&](const floatx16& s, float lsc, uint32_t (&pk)[8]) {
    const float nm = -m;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], lsc, nm));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], lsc, nm));
      pk[r >> 1] = pack2(e0, e1);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[r >> 1]), BF16_ONES, lsum, false);
    }
  };
  // O^T += V^T P^T over one 32-key half (Vh: that half of the V tile).  The
  // lane's 8 probabilities of step ks are keys 16 ks + 4 hi + 0..3 and
  // 16 ks + 8 + 4 hi + 0..3 of the half; two transpose reads give column
  // 32 dt + col of the same keys: lane a of each 16-lane group addresses key
  // (a / 4) of the four and columns 4 (a % 4) .. + 3 of the group's sixteen.
  // Rows 16 ks + 8 j + tr_row share tr_row's swizzle, so one offset per 32
  // columns serves all four reads of a column block (the rest is immediate).
  int tr_off[DT];
  {
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int cc = 32 * dt + tr_col;
      tr_off[dt] = vtoff<DG>(tr_row, cc >> 3) + (cc & 7);
    }
  }
  auto pv_half = [&](const uint32_t (&pk)[8], const bf16_t* Vh) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t pf = as_bf8(make_uint4(pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 v0 = lds_read_tr16(Vh + tr_off[dt] + (16 * ks) * D);
        const uint2 v1 = lds_read_tr16(Vh + tr_off[dt] + (16 * ks + 8) * D);
        oacc[dt] = mfma32(as_bf8(make_uint4(v0.x, v0.y, v1.x, v1.y)), pf, oacc[dt]);
      }
    }
  };
  // One whole 64-key tile, unpipelined (general path and compensation): the
  // scores (already log2-domain logits when lsc = 1) of both halves, then the
  // rescale, then P V.
  auto softmax_pv = [&](floatx16 (&s)[2], const bf16_t* VLb, const bf16_t* VHb, float lsc) {
    rescale_to(fmaxf(max_half(s[0], lsc), max_half(s[1], lsc)));
    uint32_t pk[8];
    exp_half(s[0], lsc, pk);
    pv_half(pk, VLb);
    exp_half(s[1], lsc, pk);
    pv_half(pk, VHb);
  };
  auto compute_tile = [&](const bf16_t* Kb, const bf16_t* VLb, const bf16_t* VHb, int nvalid) {
    floatx16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      zero16(s[kt]);
      qk_half(s[kt], Kb, kt);
      if (nvalid < KT) mask_half(s[kt], nvalid, kt);
    }
    softmax_pv(s, VLb, VHb, sl2);
  };

  // every wave's loads issued before this point have landed, and every
  // wave is done reading the buffers the next loads overwrite
  auto sync_loads = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };
  // Software pipeline over the whole tiles, in 32-key halves (both paths).  Each half
  // step forms the scores of one half while the probabilities of the
  // previous half are exponentiated, then accumulates P V of the previous
  // half while the new half's row maximum is taken:
  //   tile n, half 0:  S(n,0) | P(n-1,1);  P(n-1,1) V(n-1,hi) | max S(n,0)
  //   tile n, half 1:  S(n,1) | P(n,0);    P(n,0) V(n,lo)     | max S(n,1)
  // So tile n reads K(n), VH(n-1) and VL(n), and meanwhile K(n+1), VH(n) and
  // VL(n+1) land in the other halves of the double buffers.
  floatx16 s0, s1;  // scores of halves 0 and 1 (s1 carries into the next tile)
  uint32_t pk[8];
  auto tile = [&](const bf16_t* Kc, const bf16_t* VLc, const bf16_t* VHp) {
    zero16(s0);
    qk_half(s0, Kc, 0);
    exp_half(s1, sl2, pk);
    pv_half(pk, VHp);
    rescale_to(max_half(s0, sl2));
    zero16(s1);
    qk_half(s1, Kc, 1);
    exp_half(s0, sl2, pk);
    pv_half(pk, VLc);
    rescale_to(max_half(s1, sl2));
  };
  // tile 0 of a pipeline: its lower half has no predecessor
  auto first_tile = [&](const bf16_t* Kc, const bf16_t* VLc) {
    zero16(s0);
    qk_half(s0, Kc, 0);
    rescale_to(max_half(s0, sl2));
    zero16(s1);
    qk_half(s1, Kc, 1);
    exp_half(s0, sl2, pk);
    pv_half(pk, VLc);
    rescale_to(max_half(s1, sl2));
  };

  if constexpr (ALIGNED) {
    const int R = p.rcount[size_t(h) * a.Cq + i];
    const int2* rg = p.ranges + (size_t(h) * a.Cq + i) * p.Rmax;
    // ---------------- selected keys, 64-aligned ranges: whole-block tiles ----
    // Every tile arrives by direct buffer->LDS loads: the lanes of a load pick
    // their source chunks so that the lane-linear LDS placement is the
    // swizzled layout.  A load is the buffer resource (SGPRs) plus one byte
    // offset per lane; a lane's offsets inside a tile are fixed, so only the
    // tile base is added per load.
    const bf16_t* vrh = (const bf16_t*)a.v_perm + size_t(h) * N * D;
    int ri = 0, pos = R > 0 ? rg[0].x : 0, rend = R > 0 ? rg[0].y : 0;
    // the range after the current one, loaded one range ahead
    int2 rnext = R > 1 ? const_load_int2(rg, 1) : make_int2(0, 0);
    const int kbytes = int(uint32_t(N) * (D * 2)), vbytes = kbytes;
    uint32_t koff[CK], voff[CH];
#pragma unroll
    for (int q = 0; q < CK; ++q) {
      const int sl = (4 * q + w) * 64 + lane;  // K tile chunk of this lane's q-th load
      const int r = sl / DG, kc = (sl % DG) ^ swz<DG>(r);
      koff[q] = uint32_t(r * D + kc * 8) * 2;
    }
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int sl = (4 * q + w) * 64 + lane;  // V half-tile chunk
      const int r = sl / DG, c = (sl % DG) ^ vswz<DG>(r);
      voff[q] = uint32_t(r * D + c * 8) * 2;
    }
    auto issue_k = [&](bf16_t* Kd, int pos0, int nvalid) {
      const uint32_t kb = uint32_t(pos0) * (D * 2);
      if (nvalid == KT) {
#pragma unroll
        for (int q = 0; q < CK; ++q)
          buf_load_lds16(kh, kbytes, Kd + (4 * q + w) * 512, kb + koff[q]);
      } else {
        // partial tile: rows past the end of the range repeat its last row
        // (their scores are masked), so no load leaves the head's keys
#pragma unroll
        for (int q = 0; q < CK; ++q) {
          const int r = ((4 * q + w) * 64 + lane) / DG;
          const int dr = min(r, nvalid - 1) - r;
          buf_load_lds16(kh, kbytes, Kd + (4 * q + w) * 512,
                         kb + koff[q] + uint32_t(dr * D * 2));
        }
      }
    };
    // half kt (0: keys 0..31, 1: keys 32..63) of the V rows of the tile at
    // pos0 (rows past N read as zeros: the buffer's bound)
    auto issue_v = [&](bf16_t* Vd, int pos0, int kt) {
      const uint32_t vb = uint32_t(pos0 + HK * kt) * (D * 2);
#pragma unroll
      for (int q = 0; q < CH; ++q)
        buf_load_lds16(vrh, vbytes, Vd + (4 * q + w) * 512, vb + voff[q]);
    };
    // Move the cursor to the next whole 64-key tile.  False once the ranges
    // are done, or when the next tile is partial: only the last tile of a
    // range ending at N can be, and it is kept aside as the tail.
    bool have_tail = false;
    int tail_pos = 0, tail_nv = 0;
    auto next_full = [&]() -> bool {
      pos += KT;
      if (pos >= rend) {
        if (++ri >= R) return false;
        pos = rnext.x;
        rend = rnext.y;
        if (ri + 1 < R) rnext = const_load_int2(rg, ri + 1);
      }
      if (rend - pos < KT) {
        have_tail = true;
        tail_pos = pos;
        tail_nv = rend - pos;
        return false;
      }
      return true;
    };
    if (R > 0 && rend - pos < KT) {
      have_tail = true;
      tail_pos = pos;
      tail_nv = rend - pos;
    } else if (R > 0) {
      int pn = pos;
      issue_k(K0, pn, KT);
      issue_v(VL0, pn, 0);
      bool more = next_full();
      sync_loads();
      if (more) {
        issue_k(K1, pos, KT);
        issue_v(VL1, pos, 0);
      }
      issue_v(VH0, pn, 1);
      first_tile(K0, VL0);
      bool last_odd = false;  // parity of the last tile
      while (more) {
        pn = pos;
        more = next_full();
        sync_loads();
        if (more) {
          issue_k(K0, pos, KT);
          issue_v(VL0, pos, 0);
        }
        issue_v(VH1, pn, 1);
        tile(K1, VL1, VH0);
        if (!more) {
          last_odd = true;
          break;
        }
        pn = pos;
        more = next_full();
        sync_loads();
        if (more) {
          issue_k(K1, pos, KT);
          issue_v(VL1, pos, 0);
        }
        issue_v(VH0, pn, 1);
        tile(K0, VL0, VH1);
      }
      // drain: P V of the last tile's upper half
      sync_loads();
      exp_half(s1, sl2, pk);
      pv_half(pk, last_odd ? VH1 : VH0);
    }
    if (have_tail) {
      // the partial last tile, unpipelined (every buffer is free after the
      // barrier)
      __syncthreads();
      issue_k(K0, tail_pos, tail_nv);
      issue_v(VL0, tail_pos, 0);
      issue_v(VH0, tail_pos, 1);
      sync_loads();
      compute_tile(K0, VL0, VH0, tail_nv);
    }
  } else {
    // ---------------- selected keys, general ranges: row gather --------------
    const bf16_t* vh = (const bf16_t*)a.v_perm + size_t(h) * N * D;
    const int hbytes = int(uint32_t(N) * (D * 2));
    const uint32_t* mrow = a.mask + (size_t(h) * a.Cq + i) * p.W;
    const int32_t* kof = a.k_off + size_t(h) * (a.Ck + 1);
    int scan_word = 0;
    while (true) {
      __syncthreads();
      if (tid == 0) S.fsh[0] = scan_word;
      __syncthreads();
      const int nrc = fill_chunk(mrow, p.W, a.Ck, kof, S.rs, S.rp, S.wsum, S.fsh);
      scan_word = S.fsh[0];
      if (nrc == 0) break;
      const int total = S.rp[nrc];
      // Wave 0 lists the key row of every position of tile t in
      // S.rowidx[t % 3].  Window: the 64 ranges from r0, the range holding the
      // tile's first position; ranges are never empty, so they cover the
      // tile.  Short ranges: lane l writes the positions range r0 + l shares
      // with the tile.  When some range covers more than 8 of them, lane j
      // instead finds the range of position j by binary search in the window.
      // r0 then moves to the range holding the next tile's start.
      int r0 = 0;
      auto build_rows = [&](int t) {
        const int base = t * KT, end = min(base + KT, total);
        const int r = r0 + lane;
        int st = 0, en = 0;
        if (r < nrc) {
          st = S.rp[r];
          en = S.rp[r + 1];
        }
        const int lo = max(st, base), hi = min(en, end);
        int* ri = S.rowidx[t % 3];
        if (__ballot(r < nrc && hi - lo > 8)) {
          const int pos = base + lane;
          if (pos < end) {
            int L = r0, R = min(r0 + 64, nrc);  // S.rp[L] <= pos < S.rp[R]
            while (R - L > 1) {
              const int mid = (L + R) >> 1;
              if (S.rp[mid] <= pos) L = mid;
              else R = mid;
            }
            ri[lane] = S.rs[L] + (pos - S.rp[L]);
          }
        } else if (r < nrc) {
          const int rsr = S.rs[r];
          for (int pos = lo; pos < hi; ++pos) ri[pos - base] = rsr + (pos - st);
        }
        const uint64_t bal = __ballot(r < nrc && st <= base + KT);
        r0 += 63 - __clzll((unsigned long long)bal);
      };
      // K rows of tile t, and half kt of its V rows, by direct buffer->LDS
      // loads: lane l of a load lands at slot 64 q' + l of the tile, i.e. at
      // (row, chunk), and fetches the chunk the swizzled layout keeps there
      // from the listed key row.  Positions past nv repeat the last listed
      // row (their scores are masked and their probabilities are zero).
      auto issue_k = [&](bf16_t* Kd, int t, int nv) {
        const int* ri = S.rowidx[t % 3];
#pragma unroll
        for (int q = 0; q < CK; ++q) {
          const int sl = (4 * q + w) * 64 + lane;
          const int r = sl / DG, c = (sl % DG) ^ swz<DG>(r);
          const uint32_t row = uint32_t(ri[min(r, nv - 1)]);
          buf_load_lds16(kh, hbytes, Kd + (4 * q + w) * 512, row * (D * 2) + uint32_t(c * 16));
        }
      };
      auto issue_v = [&](bf16_t* Vd, int t, int kt, int nv) {
        const int* ri = S.rowidx[t % 3];
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          const int sl = (4 * q + w) * 64 + lane;  // slot in the half tile
          const int rh = sl / DG, c = (sl % DG) ^ vswz<DG>(rh);
          const uint32_t row = uint32_t(ri[min(HK * kt + rh, nv - 1)]);
          buf_load_lds16(vh, hbytes, Vd + (4 * q + w) * 512, row * (D * 2) + uint32_t(c * 16));
        }
      };
      // The whole tiles run the aligned path's pipeline.  Wave 0 lists tile
      // n + 1's rows before the barrier that precedes its loads; tile n's
      // list is still read after that barrier (its upper V half), and tile
      // n - 1's slot is free by then, hence three slots.
      const int nfull = total / KT, tail_nv = total - nfull * KT;
      if (nfull > 0) {
        if (w == 0) build_rows(0);
        __syncthreads();
        issue_k(K0, 0, KT);
        issue_v(VL0, 0, 0, KT);
        bool more = nfull > 1;
        if (w == 0 && more) build_rows(1);
        sync_loads();
        if (more) {
          issue_k(K1, 1, KT);
          issue_v(VL1, 1, 0, KT);
        }
        issue_v(VH0, 0, 1, KT);
        first_tile(K0, VL0);
        bool last_odd = false;  // parity of the last tile
        int n = 1;
        while (more) {
          more = n + 1 < nfull;
          if (w == 0 && more) build_rows(n + 1);
          sync_loads();
          if (more) {
            issue_k(K0, n + 1, KT);
            issue_v(VL0, n + 1, 0, KT);
          }
          issue_v(VH1, n, 1, KT);
          tile(K1, VL1, VH0);
          ++n;
          if (!more) {
            last_odd = true;
            break;
          }
          more = n + 1 < nfull;
          if (w == 0 && more) build_rows(n + 1);
          sync_loads();
          if (more) {
            issue_k(K1, n + 1, KT);
            issue_v(VL1, n + 1, 0, KT);
          }
          issue_v(VH0, n, 1, KT);
          tile(K0, VL0, VH1);
          ++n;
        }
        // drain: P V of the last tile's upper half
        sync_loads();
        exp_half(s1, sl2, pk);
        pv_half(pk, last_odd ? VH1 : VH0);
      }
      if (tail_nv > 0) {
        // the partial last tile, unpipelined (every buffer is free after the
        // barrier)
        __syncthreads();
        if (w == 0) build_rows(nfull);
        __syncthreads();
        issue_k(K0, nfull, tail_nv);
        issue_v(VL0, nfull, 0, tail_nv);
        issue_v(VH0, nfull, 1, tail_nv);
        sync_loads();
        compute_tile(K0, VL0, VH0, tail_nv);
      }
    }
  }

  // ---------------- compensation: tiles of cluster means ----------------
  // Each 64 consecutive key clusters form one tile of pseudo keys (their
  // means kbar, vbar as bf16 rows), run through the same pipeline as the
  // selected tiles.  Pseudo key j carries the score bias ln|K_j| / scale, so
  // that the log2-domain logit is <q, kbar_j> scale log2(e) + ln|K_j| log2(e);
  // the bias is -inf where the row selected cluster j or the cluster is
  // empty.  Tiles without a live pseudo key are skipped: the barrier before
  // each tile's loads also reports whether any of its 64 biases is finite.
  if (a.compensate) {
    const uint32_t* mr = a.mask + (size_t(h) * a.Cq + i) * p.W;
    const bf16_t* kbh = p.kbh + size_t(h) * p.Ckp * D;
    const bf16_t* vbr = p.vbr + size_t(h) * p.Ckp * D;
    const int cbytes = p.Ckp * D * 2;
    const int nct = p.Ckp / KT;
    const float isc = LOG2E / sl2;  // 1 / scale
    // a query with no finite score so far: a finite running maximum far
    // below any logit keeps a dead half from forming inf - inf (the first
    // live half rescales the empty sums by 0)
    if (m == -__builtin_huge_valf()) m = -1e30f;
    uint32_t ckoff[CK], cvoff[CH];
#pragma unroll
    for (int q = 0; q < CK; ++q) {
      const int sl = (4 * q + w) * 64 + lane;
      const int r = sl / DG, kc = (sl % DG) ^ swz<DG>(r);
      ckoff[q] = uint32_t(r * D + kc * 8) * 2;
    }
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int sl = (4 * q + w) * 64 + lane;
      const int r = sl / DG, c = (sl % DG) ^ vswz<DG>(r);
      cvoff[q] = uint32_t(r * D + c * 8) * 2;
    }
    auto issue_ck = [&](bf16_t* Kd, int t) {
      const uint32_t b = uint32_t(t * KT) * (D * 2);
#pragma unroll
      for (int q = 0; q < CK; ++q) buf_load_lds16(kbh, cbytes, Kd + (4 * q + w) * 512, b + ckoff[q]);
    };
    auto issue_cv = [&](bf16_t* Vd, int t, int kt) {
      const uint32_t b = uint32_t(t * KT + HK * kt) * (D * 2);
#pragma unroll
      for (int q = 0; q < CH; ++q) buf_load_lds16(vbr, cbytes, Vd + (4 * q + w) * 512, b + cvoff[q]);
    };
    // the biases of tile t into slot sl; 1 if one of them is finite
    auto comp_bias = [&](int t, int sl) -> int {
      int fin = 0;
      if (tid < KT) {
        const int jj = t * KT + tid;
        float b = -__builtin_huge_valf();
        if (jj < a.Ck && !((mr[jj >> 5] >> (jj & 31)) & 1u)) b = p.logsz[size_t(h) * p.Ckp + jj];
        fin = b != -__builtin_huge_valf();
        S.cbias[sl][tid] = b * isc;
      }
      return fin;
    };
    // Waits for this wave's loads, then takes the barrier that precedes the
    // next loads; it also finds the first live tile from t on (nct if none),
    // whose biases are then in slot sl.  A slot is written before that
    // barrier and read after the next one, so three slots rotate.
    auto next_live = [&](int t, int sl) -> int {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      while (!__syncthreads_or(t < nct ? comp_bias(t, sl) : 1)) ++t;
      return t;
    };
    // the scores of a half start from its biases: the MFMAs accumulate onto them
    auto bias16 = [&](floatx16& sc, const float* cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 bv = *reinterpret_cast<const float4*>(cb + 8 * g + 4 * hi);
        sc[4 * g] = bv.x;
        sc[4 * g + 1] = bv.y;
        sc[4 * g + 2] = bv.z;
        sc[4 * g + 3] = bv.w;
      }
    };
    // the selected pipeline's tile step, scores starting from the biases
    auto ctile = [&](const bf16_t* Kc, const bf16_t* VLc, const bf16_t* VHp, const float* cb) {
      bias16(s0, cb);
      qk_half(s0, Kc, 0);
      exp_half(s1, sl2, pk);
      pv_half(pk, VHp);
      rescale_to(max_half(s0, sl2));
      bias16(s1, cb + HK);
      qk_half(s1, Kc, 1);
      exp_half(s0, sl2, pk);
      pv_half(pk, VLc);
      rescale_to(max_half(s1, sl2));
    };
    auto cfirst = [&](const bf16_t* Kc, const bf16_t* VLc, const float* cb) {
      bias16(s0, cb);
      qk_half(s0, Kc, 0);
      rescale_to(max_half(s0, sl2));
      bias16(s1, cb + HK);
      qk_half(s1, Kc, 1);
      exp_half(s0, sl2, pk);
      pv_half(pk, VLc);
      rescale_to(max_half(s1, sl2));
    };
    // the first barrier also ends every wave's reads of the selected tiles
    int tc = next_live(0, 0);
    if (tc < nct) {
      issue_ck(K0, tc);
      issue_cv(VL0, tc, 0);
      int tn = next_live(tc + 1, 1);
      if (tn < nct) {
        issue_ck(K1, tn);
        issue_cv(VL1, tn, 0);
      }
      issue_cv(VH0, tc, 1);
      cfirst(K0, VL0, S.cbias[0]);
      int o = 1;              // live ordinal of tile tn
      bool last_odd = false;  // parity of the last tile
      while (tn < nct) {
        tc = tn;
        tn = next_live(tc + 1, (o + 1) % 3);
        if (tn < nct) {
          issue_ck(K0, tn);
          issue_cv(VL0, tn, 0);
        }
        issue_cv(VH1, tc, 1);
        ctile(K1, VL1, VH0, S.cbias[o % 3]);
        ++o;
        if (tn >= nct) {
          last_odd = true;
          break;
        }
        tc = tn;
        tn = next_live(tc + 1, (o + 1) % 3);
        if (tn < nct) {
          issue_ck(K1, tn);
          issue_cv(VL1, tn, 0);
        }
        issue_cv(VH0, tc, 1);
        ctile(K0, VL0, VH1, S.cbias[o % 3]);
        ++o;
      }
      // drain: P V of the last tile's upper half
      sync_loads();
      exp_half(s1, sl2, pk);
      pv_half(pk, last_odd ? VH1 : VH0);
    }
  }

  // ---------------- epilogue: normalise, stage, scatter to original rows ----
  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  // the normaliser: sum 2^(s sl2) = 2^m ltot, as a natural log
  if (a.lse && qv && hi == 0)
    a.lse[size_t(h) * N + a.q_idx[size_t(h) * N + p0 + qr]] =
        ltot > 0.f ? (m + __log2f(ltot)) * 0.69314718055994531f : -__builtin_huge_valf();
  __syncthreads();
  // stage O in the K tiles (query rows 0..63 in K0, 64..127 in K1), then
  // scatter whole rows to their original tokens
  bf16_t* Ob = w < 2 ? K0 : K1;
  const int orow = qr & 63;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * dt + 8 * g + 4 * hi;
      const uint2 v = make_uint2(pack2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                                 pack2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv));
      *reinterpret_cast<uint2*>(Ob + toff<DG>(orow, c >> 3) + (c & 7)) = v;
    }
  __syncthreads();
  const int32_t* qi = a.q_idx + size_t(h) * N + p0;
  bf16_t* oh = (bf16_t*)a.o + size_t(h) * N * D;
  for (int v = tid; v < TQ * DG; v += 256) {
    const int r = v / DG, kc = v % DG;
    if (r < nr)
      *reinterpret_cast<uint4*>(oh + size_t(qi[r]) * D + kc * 8) =
          *reinterpret_cast<const uint4*>((r < 64 ? K0 : K1) + toff<DG>(r & 63, kc));
  }
}

Prep carve(const AttnArgs& a, Arena& s) {
  Prep p{};
  const int rows = a.tile_rows;
  p.maxT = a.max_tiles > 0 ? a.max_tiles : a.N / rows + a.Cq + 1;
  p.Rmax = a.Ck <= ALIGNED_MAX_CK ? a.Ck / 2 + 1 : 0;
  p.Ckp = ceil_div(a.Ck, KT) * KT;
  p.W = ceil_div(a.Ck, 32);
  p.tiles = s.get<int4>(size_t(a.H) * p.maxT);
  p.ntiles = s.get<int32_t>(size_t(a.H));
  p.ranges = p.Rmax ? s.get<int2>(size_t(a.H) * a.Cq * p.Rmax) : nullptr;
  p.rcount = s.get<int32_t>(size_t(a.H) * a.Cq);
  p.raligned = s.get<int32_t>(size_t(a.H) * a.Cq);
  p.korder = p.Rmax ? s.get<int32_t>(size_t(a.H) * a.Ck) : nullptr;
  p.krange = p.Rmax ? s.get<int2>(size_t(a.H) * a.Ck) : nullptr;
  if (a.compensate) {
    p.logsz = s.get<float>(size_t(a.H) * p.Ckp);
    if (a.dtype == SA_BF16) {
      p.kbh = s.get<bf16_t>(size_t(a.H) * p.Ckp * a.d);
      p.vbr = s.get<bf16_t>(size_t(a.H) * p.Ckp * a.d);
    } else {
      p.kbf = s.get<float>(size_t(a.H) * p.Ckp * a.d);
      p.vbf = s.get<float>(size_t(a.H) * p.Ckp * a.d);
    }
  }
  return p;
}

}  // namespace

size_t attn_scratch(int H, int N, int d, int Cq, int Ck, int tile_rows, int compensate, int dtype,
                    int max_tiles) {
  AttnArgs a{};
  a.max_tiles = max_tiles;
  a.H = H;
  a.N = N;
  a.d = d;
  a.Cq = Cq;
  a.Ck = Ck;
  a.tile_rows = tile_rows;
  a.compensate = compensate;
  a.dtype = dtype;
  Arena s{nullptr, 0, 0};
  carve(a, s);
  return s.used;
}

hipError_t attn_run(const AttnArgs& a, Arena& s, hipStream_t st) {
  const Prep p = carve(a, s);
  if (p.Rmax) {
    key_rank_kernel<<<a.H, RANK_THREADS, 0, st>>>(a.mask, a.k_off, a.Cq, a.Ck, p.W, p.korder, p.krange);
    ranges_kernel<<<dim3(a.Cq, a.H), 64, 0, st>>>(a.mask, a.k_off, a.Cq, a.Ck, p.W, p.Rmax, a.N, p.korder,
                                                  p.krange, p.ranges, p.rcount, p.raligned);
  }
  else
    fill_zero_kernel<<<ceil_div(a.H * a.Cq, 256), 256, 0, st>>>(p.raligned, a.H * a.Cq);
  tiles_kernel<<<a.H, 1024, 0, st>>>(a.q_off, a.Cq, a.tile_rows, p.maxT, p.tiles, p.ntiles);
  if (a.compensate)
    comp_prep_kernel<<<dim3(p.Ckp, a.H), 128, 0, st>>>(a.kbar, a.vbar, a.k_off, a.Ck, p.Ckp, a.d,
                                                       p.kbh, p.vbr, p.kbf, p.vbf, p.logsz);
  const int grid = 8 * a.H * ceil_div(p.maxT, 8);
  const float sl2 = a.scale * LOG2E;
  // the caller's timing events bracket the attention kernels only (prep excluded)
  if (a.ev_start && hipEventRecord(a.ev_start, st) != hipSuccess) return hipErrorInvalidValue;
  if (a.dtype == SA_BF16) {
    if (a.d == 128) {
      if (p.Rmax) attn_mfma<128, true><<<grid, 256, 0, st>>>(a, p, sl2);
      attn_mfma<128, false><<<grid, 256, 0, st>>>(a, p, sl2);
    } else {
      if (p.Rmax) attn_mfma<64, true><<<grid, 256, 0, st>>>(a, p, sl2);
      attn_mfma<64, false><<<grid, 256, 0, st>>>(a, p, sl2);
    }
  } else {
    if (a.d == 128)
      attn_simple<float, 128><<<grid, 128, 0, st>>>(a, p, a.scale);
    else
      attn_simple<float, 64><<<grid, 128, 0, st>>>(a, p, a.scale);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.ev_stop && hipEventRecord(a.ev_stop, st) != hipSuccess) e = hipErrorInvalidValue;
  return e;
}

}  // namespace sa
