// Backward of the block-sparse attention without compensation: the gradients
// of Q, K and V given the output gradient dO, over the same selected key
// clusters as the forward (the trainable use of block-sparse attention:
// "Bidirectional Sparse Attention for Faster Video Diffusion Training",
// abstract; "VMoBA: Mixture-of-Block Attention for Video Diffusion Models",
// English abstract).  For a query n of query cluster i and a key m of a key
// cluster it selected, with s_nm = <q_n, k_m> scale and P_nm = softmax_m s_nm:
//   dV_m += P_nm dO_n,   dP_nm = <dO_n, v_m>,   D_n = sum_m P_nm dP_nm
//   dS_nm = P_nm (dP_nm - D_n),   dQ_n = scale sum_m dS_nm k_m,
//   dK_m += scale sum_n dS_nm q_n.
// D_n is taken as <dO_n, O_n> with the forward's output (the two are equal).
//
// Kernels (bf16 inputs, fp32 gradients in original token order):
//  * prep: dO rows in query-cluster order, D per query, and for every key
//    cluster the list of query clusters that selected it (ascending);
//  * dq: one workgroup of 4 wavefronts per query tile (<= 128 rows, 32 per
//    wavefront, one query column per lane as in the forward); pass 1 forms
//    the log-sum-exp of every query over its selected keys, pass 2 forms P,
//    dP^T = V dO^T, dS^T and dQ^T += K^T dS^T on 32x32x16 bf16 MFMA, walking
//    the selected key clusters in 32-key steps;
//  * dkdv: one workgroup of 4 wavefronts per block of <= 128 keys of one key
//    cluster (32 keys per wavefront, one key column per lane), walking the
//    query clusters that selected it in 32-query steps: S = Q K^T,
//    dP = dO V^T, dV^T += dO^T P and dK^T += Q^T dS.
// Every sum runs in a fixed order (no atomics): results are deterministic.

#include "sa_internal.h"

namespace sa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr int TB = 32;        // rows per MFMA block (keys or queries)
constexpr int QT = 128;       // query rows per dq workgroup (4 wavefronts)
constexpr int KB = 128;       // keys per dkdv workgroup (4 wavefronts)
constexpr float LOG2E = 1.4426950408889634f;
constexpr int BUF_DWORD3 = 0x00020000;

__device__ __forceinline__ floatx16 mfma32(bf16x8_t a, bf16x8_t b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t as_bf8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_t __attribute__((address_space(3)))*)p);
  return __builtin_bit_cast(uint2, r);
}
// 16 bytes per lane from a raw buffer over [base, base + nbytes) into LDS
// (lane l lands at lds + 16 l; offsets past the end read zeros).  nbytes is
// the unsigned 32-bit record count carried in an int (up to 2^32 - 1).
__device__ __forceinline__ void buf_load_lds16(const void* base, int nbytes, bf16_t* lds, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nbytes, BUF_DWORD3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, 0);
}
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

// LDS tile of 32 rows x D bf16, rows of D/8 16-byte chunks XOR-swizzled by
// 2 (row mod CPR/2): conflict-free for the transpose reads and at most 2-way
// for whole-row chunk reads.
template <int CPR>
__device__ __forceinline__ int toff(int r, int c) {
  return r * (CPR * 8) + ((c ^ ((r & (CPR / 2 - 1)) << 1)) << 3);
}

// Load rows [row0, row0 + 32) of a [N, D] bf16 matrix into an LDS tile
// (rows past `valid` repeat row valid-1, so nothing reads outside the
// matrix; their values are masked by the caller).  All 256 threads.
template <int D>
__device__ __forceinline__ void load_tile(const bf16_t* base, int nbytes, bf16_t* tile, int row0, int valid) {
  constexpr int DG = D / 8;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
#pragma unroll
  for (int q = 0; q < (TB * DG) / 256; ++q) {
    const int sl = (4 * q + w) * 64 + lane;       // slot in the tile, lane-linear
    const int r = sl / DG, cs = sl % DG;          // LDS row and chunk position
    const int c = cs ^ ((r & (DG / 2 - 1)) << 1);  // source chunk kept there
    const int src = row0 + min(r, valid - 1);
    buf_load_lds16(base, nbytes, tile + (4 * q + w) * 512, uint32_t(src * D + c * 8) * 2u);
  }
}

// A operand from a row-major LDS tile: row (lane % 32), d = 16 st + 8 hi .. + 7
template <int D>
__device__ __forceinline__ bf16x8_t frag_rows(const bf16_t* tile, int st) {
  constexpr int DG = D / 8;
  const int lane = threadIdx.x & 63, col = lane & 31, hi = lane >> 5;
  return as_bf8(*reinterpret_cast<const uint4*>(tile + toff<DG>(col, 2 * st + hi)));
}

// A operand of X^T (d x rows): d row 32 dt + (lane % 32), the 8 rows of
// k-step ks that a D-layout result's lane holds (16 ks + 4 hi + 0..3 and
// 16 ks + 8 + 4 hi + 0..3), by two LDS transpose reads.
template <int D>
__device__ __forceinline__ bf16x8_t frag_tr(const bf16_t* tile, int dt, int ks) {
  constexpr int DG = D / 8;
  const int lane = threadIdx.x & 63, hi = lane >> 5;
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int cc = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int off = toff<DG>(tr_row, cc >> 3) + (cc & 7);
  const uint2 v0 = lds_read_tr16(tile + off + (16 * ks) * D);
  const uint2 v1 = lds_read_tr16(tile + off + (16 * ks + 8) * D);
  return as_bf8(make_uint4(v0.x, v0.y, v1.x, v1.y));
}

// row r of the D layout held by element e of a lane (rows 8 (e / 4) + 4 hi + e % 4)
__device__ __forceinline__ int drow(int e, int hi) { return 8 * (e >> 2) + 4 * hi + (e & 3); }

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
// dO rows into query-cluster order, and D = <dO, O> per query (fp32, fixed
// order).  One wavefront per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16_t* __restrict__ dO, const bf16_t* __restrict__ O,
                                                       const int32_t* __restrict__ q_idx, int H, int N,
                                                       bf16_t* __restrict__ dO_perm, float* __restrict__ Dv) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (long long)H * N) return;
  const int h = int(row / N);
  const long long src = (long long)h * N + q_idx[row];
  float acc = 0.f;
  for (int c = lane; c < D; c += 64) {
    const bf16_t g = dO[src * D + c];
    dO_perm[row * D + c] = g;
    acc = fmaf(bf2f(g), bf2f(O[src * D + c]), acc);
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) Dv[row] = acc;
}

// For every (head, key cluster j): the query clusters i whose mask row sets
// j, ascending.  One thread per (head, j).
__global__ void bwd_transpose_kernel(const uint32_t* __restrict__ mask, int H, int Cq, int Ck,
                                     int32_t* __restrict__ tcount, int32_t* __restrict__ tlist) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)H * Ck) return;
  const int h = int(idx / Ck), j = int(idx % Ck);
  const int W = ceil_div(Ck, 32);
  int32_t* out = tlist + idx * Cq;
  int n = 0;
  for (int i = 0; i < Cq; ++i)
    if ((mask[(size_t(h) * Cq + i) * W + (j >> 5)] >> (j & 31)) & 1u) out[n++] = i;
  tcount[idx] = n;
}

// tiles of <= `rows` consecutive rows inside each cluster: {cluster, first row, rows}
__global__ __launch_bounds__(1024) void bwd_tiles_kernel(const int32_t* __restrict__ off, int C, int rows,
                                                         int maxT, int4* __restrict__ tiles,
                                                         int32_t* __restrict__ ntiles) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int h = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int32_t* o = off + size_t(h) * (C + 1);
  if (t == 0) carry = 0;
  __syncthreads();
  for (int b = 0; b < C; b += 1024) {
    const int i = b + t;
    const int sz = i < C ? o[i + 1] - o[i] : 0;
    const int nt = ceil_div(sz, rows);
    int x = nt;
    for (int k = 1; k < 64; k <<= 1) {
      const int y = __shfl_up(x, k, 64);
      if (lane >= k) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int pre = carry;
    for (int j = 0; j < w; ++j) pre += wsum[j];
    pre += x - nt;
    for (int u = 0; u < nt; ++u)
      if (pre + u < maxT) tiles[size_t(h) * maxT + pre + u] = make_int4(i, o[i] + u * rows, min(rows, sz - u * rows), 0);
    __syncthreads();
    if (t == 1023) carry = pre + nt;
    __syncthreads();
  }
  if (t == 0) ntiles[h] = carry;
}

// ---------------------------------------------------------------------------
// dq: one workgroup per query tile
// ---------------------------------------------------------------------------
struct BwdArgs {
  int H, N, Cq, Ck, maxTq, maxTk;
  float scale;
  const bf16_t* q_perm;   // [H][N][D] query-cluster order
  const int32_t* q_idx;   // [H][N] original index of each query position
  const int32_t* q_off;   // [H][Cq+1]
  const bf16_t* k_perm;   // [H][N][D] key-cluster order
  const int32_t* k_idx;   // [H][N] original index of each key position
  const int32_t* k_off;   // [H][Ck+1]
  const bf16_t* v_perm;   // [H][N][D] key-cluster order
  const uint32_t* mask;   // [H][Cq][W]
  const bf16_t* dO_perm;  // [H][N][D] query-cluster order
  const float* lse_in;    // [H][N] original order, the forward's natural-log normaliser (optional)
  const float* Dv;        // [H][N] query-cluster order
  float* lse2;            // [H][N] log2-domain log-sum-exp, query-cluster order
  const int4* qtiles;     // [H][maxTq]
  const int32_t* nqt;     // [H]
  const int4* ktiles;     // [H][maxTk]
  const int32_t* nkt;     // [H]
  const int32_t* tcount;  // [H][Ck]
  const int32_t* tlist;   // [H][Ck][Cq]
  float* dq;              // [H][N][D] fp32, original order
  float* dk;
  float* dv;
};

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int DS = D / 16, DT = D / 32;
  // a step covers up to SBK 32-key blocks behind one load and barrier
  constexpr int SBK = 2;
  __shared__ __attribute__((aligned(16))) bf16_t Kt[SBK * TB * D];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[SBK * TB * D];
  const int h = blockIdx.y, tix = blockIdx.x;
  if (tix >= a.nqt[h]) return;
  const int4 td = a.qtiles[size_t(h) * a.maxTq + tix];
  const int i = td.x, p0 = td.y, nr = td.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int qr = 32 * w + col;            // this lane's query row in the tile
  const bool qv = qr < nr;
  const size_t qpos = size_t(h) * N + p0 + (qv ? qr : 0);
  // B operands: Q^T and dO^T of the lane's query, d = 16 s + 8 hi .. + 7
  bf16x8_t qf[DS], gf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 u = *reinterpret_cast<const uint4*>(a.q_perm + qpos * D + 16 * s + 8 * hi);
    uint4 g = *reinterpret_cast<const uint4*>(a.dO_perm + qpos * D + 16 * s + 8 * hi);
    if (!qv) u = g = make_uint4(0, 0, 0, 0);
    qf[s] = as_bf8(u);
    gf[s] = as_bf8(g);
  }
  const float sl2 = a.scale * LOG2E;
  const int kbytes = int(uint32_t(N) * (D * 2));
  const bf16_t* kh = a.k_perm + size_t(h) * N * D;
  const bf16_t* vh = a.v_perm + size_t(h) * N * D;
  const int32_t* ko = a.k_off + size_t(h) * (a.Ck + 1);
  const uint32_t* mr = a.mask + (size_t(h) * a.Cq + i) * size_t(ceil_div(a.Ck, 32));
  const int W = ceil_div(a.Ck, 32);

  // S^T of one 32-key step (keys of this step past `nv` -> -inf)
  auto scores = [&](floatx16& s, const bf16_t* Kb, int nv) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int st = 0; st < DS; ++st) s = mfma32(frag_rows<D>(Kb, st), qf[st], s);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (drow(r, hi) >= nv) s[r] = -__builtin_huge_valf();
  };
  // every selected key cluster in steps of up to SBK 32-key blocks;
  // body(K block, V block, nv) for each block after the step's tiles are in LDS
  auto walk = [&](bool with_v, auto&& body) {
    for (int wd = 0; wd < W; ++wd) {
      uint32_t bits = mr[wd];
      const int rem = a.Ck - 32 * wd;  // bits past the last key cluster are ignored
      if (rem < 32) bits &= (1u << rem) - 1u;
      while (bits) {
        const int j = 32 * wd + __ffs(bits) - 1;
        bits &= bits - 1;
        const int k0 = ko[j], k1 = ko[j + 1];
        for (int p = k0; p < k1; p += SBK * TB) {
          const int nv = min(SBK * TB, k1 - p);
          const int nb = ceil_div(nv, TB);  // blocks in this step (uniform)
          __syncthreads();  // the previous step is done with the tiles
          for (int b = 0; b < nb; ++b) {
            load_tile<D>(kh, kbytes, Kt + b * TB * D, p + b * TB, min(TB, nv - b * TB));
            if (with_v) load_tile<D>(vh, kbytes, Vt + b * TB * D, p + b * TB, min(TB, nv - b * TB));
          }
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
          __syncthreads();
          for (int b = 0; b < nb; ++b) body(Kt + b * TB * D, Vt + b * TB * D, min(TB, nv - b * TB));
        }
      }
    }
  };

  // pass 1: log-sum-exp of the lane's query (log2 domain), unless the
  // forward's is given
  float m = -__builtin_huge_valf(), l = 0.f;
  if (!a.lse_in) walk(false, [&](const bf16_t* Kb, const bf16_t*, int nv) {
    floatx16 s;
    scores(s, Kb, nv);
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx) * sl2;
    const float mn = fmaxf(m, mx);
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -mn));
    l = l * __builtin_amdgcn_exp2f(m - mn) + pair_sum(acc);
    m = mn;
  });
  float lse = l > 0.f ? m + __log2f(l) : __builtin_huge_valf();  // no key: P = 0
  if (a.lse_in) {
    const float ln = qv ? a.lse_in[size_t(h) * N + a.q_idx[qpos]] : 0.f;
    lse = ln == -__builtin_huge_valf() ? __builtin_huge_valf() : ln * LOG2E;
  }
  const float dn = qv ? a.Dv[qpos] : 0.f;
  if (qv && hi == 0) a.lse2[qpos] = lse;

  // pass 2: dQ^T += K^T dS^T
  floatx16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  walk(true, [&](const bf16_t* Kb, const bf16_t* Vb, int nv) {
    floatx16 s, dp;
    scores(s, Kb, nv);
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
    for (int st = 0; st < DS; ++st) dp = mfma32(frag_rows<D>(Vb, st), gf[st], dp);  // dP^T = V dO^T
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0v = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse));
      const float p1v = __builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -lse));
      pk[r >> 1] = pack2(p0v * (dp[r] - dn), p1v * (dp[r + 1] - dn));  // dS^T
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t bf = as_bf8(make_uint4(pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(frag_tr<D>(Kb, dt, ks), bf, acc[dt]);
    }
  });
  // lane (col, hi) holds dQ^T[32 dt + drow(r)][query col]
  if (qv) {
    float* out = a.dq + (size_t(h) * N + a.q_idx[qpos]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[32 * dt + drow(r, hi)] = acc[dt][r] * a.scale;
  }
}

// ---------------------------------------------------------------------------
// dkdv: one workgroup per block of <= 128 keys of one key cluster
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int DS = D / 16, DT = D / 32;
  // a step covers up to SB 32-row blocks of query rows behind one load and
  // barrier (the kernel runs one workgroup per CU: registers, not LDS, bound it)
  constexpr int SB = 4;
  __shared__ __attribute__((aligned(16))) bf16_t Qt[SB * TB * D];
  __shared__ __attribute__((aligned(16))) bf16_t Gt[SB * TB * D];
  __shared__ float lse_s[SB * TB], d_s[SB * TB];
  const int h = blockIdx.y, tix = blockIdx.x;
  if (tix >= a.nkt[h]) return;
  const int4 td = a.ktiles[size_t(h) * a.maxTk + tix];
  const int j = td.x, p0 = td.y, nk = td.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, col = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int kr = 32 * w + col;  // this lane's key in the block
  const bool kv = kr < nk;
  const size_t kpos = size_t(h) * N + p0 + (kv ? kr : 0);
  // B operands: K^T and V^T of the lane's key
  bf16x8_t kf[DS], vf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 u = *reinterpret_cast<const uint4*>(a.k_perm + kpos * D + 16 * s + 8 * hi);
    uint4 v = *reinterpret_cast<const uint4*>(a.v_perm + kpos * D + 16 * s + 8 * hi);
    if (!kv) u = v = make_uint4(0, 0, 0, 0);
    kf[s] = as_bf8(u);
    vf[s] = as_bf8(v);
  }
  const float sl2 = a.scale * LOG2E;
  const int qbytes = int(uint32_t(N) * (D * 2));
  const bf16_t* qh = a.q_perm + size_t(h) * N * D;
  const bf16_t* gh = a.dO_perm + size_t(h) * N * D;
  const int32_t* qo = a.q_off + size_t(h) * (a.Cq + 1);
  const size_t jj = size_t(h) * a.Ck + j;
  const int nsel = a.tcount[jj];
  const int32_t* lst = a.tlist + jj * a.Cq;
  floatx16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[dt][r] = dva[dt][r] = 0.f;
  // one 32-row block of the step: S = Q K^T (rows queries, lane column =
  // key), dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS
  auto block = [&](const bf16_t* Qb, const bf16_t* Gb, const float* lse_b, const float* d_b) {
    floatx16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      s = mfma32(frag_rows<D>(Qb, st), kf[st], s);
      dp = mfma32(frag_rows<D>(Gb, st), vf[st], dp);
    }
    uint32_t pp[8], ds[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int r0 = drow(r, hi), r1 = drow(r + 1, hi);
      // query rows past nv carry lse = +inf: P = 0
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse_b[r0]));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -lse_b[r1]));
      pp[r >> 1] = pack2(e0, e1);
      ds[r >> 1] = pack2(e0 * (dp[r] - d_b[r0]), e1 * (dp[r + 1] - d_b[r1]));
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t pb = as_bf8(make_uint4(pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]));
      const bf16x8_t db = as_bf8(make_uint4(ds[4 * ks], ds[4 * ks + 1], ds[4 * ks + 2], ds[4 * ks + 3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dva[dt] = mfma32(frag_tr<D>(Gb, dt, ks), pb, dva[dt]);  // dV^T += dO^T P
        dka[dt] = mfma32(frag_tr<D>(Qb, dt, ks), db, dka[dt]);  // dK^T += Q^T dS
      }
    }
  };
  for (int u = 0; u < nsel; ++u) {
    const int i = lst[u];
    const int q0 = qo[i], q1 = qo[i + 1];
    for (int p = q0; p < q1; p += SB * TB) {
      const int nv = min(SB * TB, q1 - p);
      const int nb = ceil_div(nv, TB);  // blocks in this step (uniform)
      __syncthreads();  // the previous step is done with the tiles
      for (int b = 0; b < nb; ++b) {
        load_tile<D>(qh, qbytes, Qt + b * TB * D, p + b * TB, min(TB, nv - b * TB));
        load_tile<D>(gh, qbytes, Gt + b * TB * D, p + b * TB, min(TB, nv - b * TB));
      }
      if (t < SB * TB) {
        const bool ok = t < nv;
        lse_s[t] = ok ? a.lse2[size_t(h) * N + p + t] : __builtin_huge_valf();
        d_s[t] = ok ? a.Dv[size_t(h) * N + p + t] : 0.f;
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      for (int b = 0; b < nb; ++b) block(Qt + b * TB * D, Gt + b * TB * D, lse_s + b * TB, d_s + b * TB);
    }
  }
  if (kv) {
    const size_t o = (size_t(h) * N + a.k_idx[kpos]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        a.dk[o + 32 * dt + drow(r, hi)] = dka[dt][r] * a.scale;
        a.dv[o + 32 * dt + drow(r, hi)] = dva[dt][r];
      }
  }
}

struct BwdPrep {
  bf16_t* dO_perm;
  float* Dv;
  float* lse2;
  int4* qtiles;
  int32_t* nqt;
  int4* ktiles;
  int32_t* nkt;
  int32_t* tcount;
  int32_t* tlist;
  int maxTq, maxTk;
};

BwdPrep carve_bwd(int H, int N, int d, int Cq, int Ck, Arena& s) {
  BwdPrep b{};
  b.maxTq = N / QT + Cq + 1;
  b.maxTk = N / KB + Ck + 1;
  b.dO_perm = s.get<bf16_t>(size_t(H) * N * d);
  b.Dv = s.get<float>(size_t(H) * N);
  b.lse2 = s.get<float>(size_t(H) * N);
  b.qtiles = s.get<int4>(size_t(H) * b.maxTq);
  b.nqt = s.get<int32_t>(size_t(H));
  b.ktiles = s.get<int4>(size_t(H) * b.maxTk);
  b.nkt = s.get<int32_t>(size_t(H));
  b.tcount = s.get<int32_t>(size_t(H) * Ck);
  b.tlist = s.get<int32_t>(size_t(H) * Ck * Cq);
  return b;
}

}  // namespace

size_t attn_bwd_scratch(int H, int N, int d, int Cq, int Ck) {
  Arena a{nullptr, 0, 0};
  carve_bwd(H, N, d, Cq, Ck, a);
  return a.used;
}

hipError_t attn_bwd_run(const AttnBwdArgs& g, Arena& s, hipStream_t st) {
  if (g.d != 64 && g.d != 128) return hipErrorInvalidValue;
  const BwdPrep b = carve_bwd(g.H, g.N, g.d, g.Cq, g.Ck, s);
  BwdArgs a{};
  a.H = g.H;
  a.N = g.N;
  a.Cq = g.Cq;
  a.Ck = g.Ck;
  a.maxTq = b.maxTq;
  a.maxTk = b.maxTk;
  a.scale = g.scale;
  a.q_perm = (const bf16_t*)g.q_perm;
  a.q_idx = g.q_idx;
  a.q_off = g.q_off;
  a.k_perm = (const bf16_t*)g.k_perm;
  a.k_idx = g.k_idx;
  a.k_off = g.k_off;
  a.v_perm = (const bf16_t*)g.v_perm;
  a.mask = g.mask;
  a.dO_perm = b.dO_perm;
  a.lse_in = g.lse;
  a.Dv = b.Dv;
  a.lse2 = b.lse2;
  a.qtiles = b.qtiles;
  a.nqt = b.nqt;
  a.ktiles = b.ktiles;
  a.nkt = b.nkt;
  a.tcount = b.tcount;
  a.tlist = b.tlist;
  a.dq = g.dq;
  a.dk = g.dk;
  a.dv = g.dv;
  const long long rows = (long long)g.H * g.N;
  const unsigned prep_grid = unsigned((rows + 3) / 4);
  if (g.d == 128)
    bwd_prep_kernel<128><<<prep_grid, 256, 0, st>>>((const bf16_t*)g.dO, (const bf16_t*)g.O, g.q_idx, g.H, g.N,
                                                    b.dO_perm, b.Dv);
  else
    bwd_prep_kernel<64><<<prep_grid, 256, 0, st>>>((const bf16_t*)g.dO, (const bf16_t*)g.O, g.q_idx, g.H, g.N,
                                                   b.dO_perm, b.Dv);
  bwd_transpose_kernel<<<unsigned((size_t(g.H) * g.Ck + 255) / 256), 256, 0, st>>>(g.mask, g.H, g.Cq, g.Ck, b.tcount,
                                                                                   b.tlist);
  bwd_tiles_kernel<<<g.H, 1024, 0, st>>>(g.q_off, g.Cq, QT, b.maxTq, b.qtiles, b.nqt);
  bwd_tiles_kernel<<<g.H, 1024, 0, st>>>(g.k_off, g.Ck, KB, b.maxTk, b.ktiles, b.nkt);
  // every gradient row is written by exactly one workgroup: the tiles cover
  // every position (a key no query selected, or a query with no selected key,
  // gets zeros)
  const dim3 gq(b.maxTq, g.H), gk(b.maxTk, g.H);
  if (g.d == 128) {
    bwd_dq_kernel<128><<<gq, 256, 0, st>>>(a);
    bwd_dkdv_kernel<128><<<gk, 256, 0, st>>>(a);
  } else {
    bwd_dq_kernel<64><<<gq, 256, 0, st>>>(a);
    bwd_dkdv_kernel<64><<<gk, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sa
