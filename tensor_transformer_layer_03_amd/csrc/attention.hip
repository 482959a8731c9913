// Flash-style self-attention over one rank's heads (podcast page, Outline and
// Key concepts: self-attention parallelised by heads, so each rank runs whole
// heads with no exchange; guide page section 3.2).
//
// Per head and sequence: O = softmax(Q K^T / sqrt(d) (+ causal mask)) V, the
// probabilities never leave registers; the row log-sum-exp is kept for the
// backward. The backward is two deterministic kernels (no atomics):
//   dK/dV: one workgroup per 128 keys, looping over query tiles;
//   dQ:    one workgroup per 128 queries, looping over key tiles.
//
// Layout trick: the forward computes S^T = K Q^T with the 32x32 MFMA, so the
// accumulator lane l owns query l%32 and 16 keys. Online-softmax statistics
// are then per lane (one cross-half shuffle, lane ^ 32), the O rescale is a
// lane-uniform multiply, and the probabilities feed O^T = V^T P^T directly as
// the MFMA B operand. The 16 keys of a lane are not contiguous, so V^T is
// stored in LDS with key positions permuted (bits 2 and 3 of the key offset
// inside each 16-key group swapped); a lane then reads its 8 keys with one
// 16-byte LDS load. The same holds for K^T (dQ) and for Q^T, dO^T (dK/dV,
// where the roles of queries and keys swap).
#include "common.h"
#include "kernels.h"

namespace tpl {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;   // largest exp2-domain growth of a row max before O is rescaled

struct Args {
  const char* qkv; int64_t ld_qkv;
  char* ctx; int64_t ld_ctx;
  float* lse;
  const char* dctx;
  char* dqkv;
  float* delta;
  int batch, heads, seq;
};

// Row tile: ROWS rows x D elements from global into LDS [ROWS][D + pad].
template <typename T, int D, int ROWS, int NT>
struct RowTile {
  static constexpr int kVec = 16 / sizeof(T);
  static constexpr int kLd = D + kVec;
  static constexpr int kCpr = D / kVec;
  static constexpr int kTotal = ROWS * kCpr;
  static constexpr int kPer = (kTotal + NT - 1) / NT;
  static_assert(NT % 64 == 0, "whole waves per workgroup");
  u32x4 r[kPer];
  // base points at element (row 0, col 0) of the head; rows >= nrows read as 0.
  __device__ __forceinline__ void load(const T* base, int64_t ld, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int idx = tid + i * NT;
      int row = idx / kCpr, c = idx % kCpr;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (idx < kTotal && row0 + row < nrows) v = ld16(base + (int64_t)(row0 + row) * ld + c * kVec);
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int idx = tid + i * NT;
      if (idx >= kTotal) break;
      int row = idx / kCpr, c = idx % kCpr;
      st16(lds + row * kLd + c * kVec, r[i]);
    }
  }
};

// Transposed tile: 64 rows x D elements from global into LDS [D][64 + pad]
// with row positions permuted within each 16-row group (bits 2,3 swapped), so
// the 8 rows {16q+4h+0..3, 16q+8+4h+0..3} land at positions 16q+8h+0..7.
template <typename T, int D, int NT>
struct TransTile {
  static constexpr int kVec = 16 / sizeof(T);
  static constexpr int kLd = 64 + kVec;
  static constexpr int kUnits = 8 * (D / kVec);
  static constexpr int kPer = (kUnits + NT - 1) / NT;
  u32x4 r[kPer][8];
  __device__ __forceinline__ static int row_of(int kg, int e) {
    const int q = kg >> 1, h = kg & 1;
    return 16 * q + (e < 4 ? 4 * h + e : 8 + 4 * h + (e - 4));
  }
  __device__ __forceinline__ void load(const T* base, int64_t ld, int row0, int nrows, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      int dv = unit % (D / kVec), kg = unit / (D / kVec);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int row = row0 + row_of(kg, e);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (unit < kUnits && row < nrows) v = ld16(base + (int64_t)row * ld + dv * kVec);
        r[u][e] = v;
      }
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      if (unit >= kUnits) break;
      int dv = unit % (D / kVec), kg = unit / (D / kVec);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          u32x4 o;
#pragma unroll
          for (int p = 0; p < 4; ++p) o[p] = __builtin_amdgcn_perm(r[u][2 * p + 1][c >> 1], r[u][2 * p][c >> 1], sel);
          st16(lds + (dv * 8 + c) * kLd + 8 * kg, o);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 lo = {r[u][0][c], r[u][1][c], r[u][2][c], r[u][3][c]};
          u32x4 hi = {r[u][4][c], r[u][5][c], r[u][6][c], r[u][7][c]};
          T* p = lds + (dv * 4 + c) * kLd + 8 * kg;
          st16(p, lo);
          st16(p + 4, hi);
        }
      }
    }
  }
};

// Fragment of 8 values taken from accumulator `acc` slots base..base+7.
template <typename T>
__device__ __forceinline__ void acc_frag(Frag8<T>& f, const f32x16& acc, int base) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = acc[base + e];
  frag_from_f32(f, v);
}

// Store a transposed accumulator tile: lane owns row `row` (query or key) and
// d = dt*32 + 8*(r/4) + 4*grp + r%4.
template <typename T, int D>
__device__ __forceinline__ void store_rows(T* base, int64_t ld, int row, const f32x16* acc, float scale, int grp) {
  T* p = base + (int64_t)row * ld;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = dt * 32 + 8 * q + 4 * grp;
      store4(p + d, acc[dt][4 * q] * scale, acc[dt][4 * q + 1] * scale, acc[dt][4 * q + 2] * scale,
             acc[dt][4 * q + 3] * scale);
    }
}

// LDS buffers per tile of the generic backward kernels: two (the next tile
// is stored while the current one is read) except for fp32 above head size
// 64, whose double-buffered tiles would exceed the 160 KB of a workgroup;
// with one buffer the store of the next tile waits for a barrier.
template <typename T, int D>
constexpr int bwd_buffers() { return sizeof(T) == 4 && D > 64 ? 1 : 2; }

// ------------------------------------------------------------------ forward
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_kernel(Args a) {
  constexpr int NT = 256, BQ = 128, BKV = 64;
  using KT = RowTile<T, D, BKV, NT>;
  using VT = TransTile<T, D, NT>;
  __shared__ __attribute__((aligned(16))) T sK[2][BKV * KT::kLd];
  __shared__ __attribute__((aligned(16))) T sVt[2][D * VT::kLd];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, grp = lane >> 5;
  // 1-D grid dealt heaviest query tiles first over all heads (causal tiles
  // differ up to seq/BQ-fold in work, so the last to start are the short ones)
  const int bhs = a.batch * a.heads, bh = blockIdx.x % bhs;
  const int qb = gridDim.x / bhs - 1 - blockIdx.x / bhs;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int s = a.seq;
  const int hr = a.heads * D;
  const T* Qg = reinterpret_cast<const T*>(a.qkv) + (int64_t)b * s * a.ld_qkv + hd * D;
  const T* Kg = Qg + hr;
  const T* Vg = Qg + 2 * hr;
  const int q0 = qb * BQ, q0w = q0 + wave * 32, my_q = q0w + l32;
  const float c = kLog2e * rsqrtf((float)D);

  Frag8<T> qf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_q < s) load_frag(qf[st], Qg + (int64_t)my_q * a.ld_qkv + st * 16 + grp * 8);
    else { float z[8] = {0, 0, 0, 0, 0, 0, 0, 0}; frag_from_f32(qf[st], z); }
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int kv_end = CAUSAL ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  KT kt_ld;
  VT vt_ld;
  kt_ld.load(Kg, a.ld_qkv, 0, s, tid);
  vt_ld.load(Vg, a.ld_qkv, 0, s, tid);
  kt_ld.store(sK[0], tid);
  vt_ld.store(sVt[0], tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1, kv0 = t * BKV;
    const bool more = t + 1 < ntiles;
    if (more) {
      kt_ld.load(Kg, a.ld_qkv, kv0 + BKV, s, tid);
      vt_ld.load(Vg, a.ld_qkv, kv0 + BKV, s, tid);
    }
    if (!CAUSAL || kv0 <= q0w + 31) {
      f32x16 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          Frag8<T> kf;
          load_frag(kf, &sK[cur][(kt * 32 + l32) * KT::kLd + st * 16 + grp * 8]);
          mfma_step(sc[kt], kf, qf[st]);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kt * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
          float v = sc[kt][r] * c;
          if (key >= s || (CAUSAL && key > my_q)) v = -INFINITY;
          sc[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(sc[kt][r] - m_use);
          sc[kt][r] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 32, kWave);
      l = l * alpha + sum;
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag8<T> pf;
        acc_frag(pf, sc[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          Frag8<T> vf;
          load_frag(vf, &sVt[cur][(dt * 32 + l32) * VT::kLd + ks * 16 + grp * 8]);
          mfma_step(o[dt], vf, pf);
        }
      }
    }
    if (more) {
      kt_ld.store(sK[cur ^ 1], tid);
      vt_ld.store(sVt[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if (my_q < s) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T* Og = reinterpret_cast<T*>(a.ctx) + (int64_t)b * s * a.ld_ctx + hd * D;
    store_rows<T, D>(Og, a.ld_ctx, my_q, o, inv, grp);
    if (grp == 0) a.lse[((int64_t)b * a.heads + hd) * s + my_q] = m * kLn2 + logf(l);
  }
}

// ------------------------------------------------------------------ backward prologue
// delta[b][h][q] = sum_d dO[q][d] * O[q][d]  (= sum_j P_qj dP_qj). A group of
// G lanes takes one (token, head): lane j reads 16-B chunk j of O and dO, so
// consecutive groups read consecutive stretches of a token's row (coalesced),
// and the G partial dots are summed with lane shuffles in a fixed tree.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(Args a) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kChunks = D / kVec;   // 16-B chunks per (token, head)
  constexpr int G = kChunks <= 8 ? 8 : (kChunks <= 16 ? 16 : 32);
  static_assert(kChunks <= G && G <= kWave, "group does not fit a wave");
  const int64_t gid = ((int64_t)blockIdx.x * 256 + threadIdx.x) / G;   // token row * heads + head
  const int j = (int)(threadIdx.x % G);
  const bool live = gid < (int64_t)a.batch * a.seq * a.heads;
  const int64_t row = gid / a.heads;
  const int hd = (int)(gid % a.heads);
  float acc = 0.f;
  if (live && j < kChunks) {
    const T* o = reinterpret_cast<const T*>(a.ctx) + row * a.ld_ctx + hd * D + j * kVec;
    const T* d = reinterpret_cast<const T*>(a.dctx) + row * a.ld_ctx + hd * D + j * kVec;
    Vec16<T> vo, vd;
    vo.raw = ld16(o);
    vd.raw = ld16(d);
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc += to_f32(vo.get(e)) * to_f32(vd.get(e));
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (live && j == 0) {
    const int64_t b = row / a.seq, q = row % a.seq;
    a.delta[(b * a.heads + hd) * a.seq + q] = acc;
  }
}

// ------------------------------------------------------------------ backward: dQ
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(Args a) {
  constexpr int NT = 256, BQ = 128, BKV = 64;
  constexpr int NB = bwd_buffers<T, D>();
  using KT = RowTile<T, D, BKV, NT>;
  using TT = TransTile<T, D, NT>;
  __shared__ __attribute__((aligned(16))) T sK[NB][BKV * KT::kLd];
  __shared__ __attribute__((aligned(16))) T sV[NB][BKV * KT::kLd];
  __shared__ __attribute__((aligned(16))) T sKt[NB][D * TT::kLd];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, grp = lane >> 5;
  // 1-D grid dealt heaviest query tiles first over all heads (causal tiles
  // differ up to seq/BQ-fold in work, so the last to start are the short ones)
  const int bhs = a.batch * a.heads, bh = blockIdx.x % bhs;
  const int qb = gridDim.x / bhs - 1 - blockIdx.x / bhs;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int s = a.seq, hr = a.heads * D;
  const T* Qg = reinterpret_cast<const T*>(a.qkv) + (int64_t)b * s * a.ld_qkv + hd * D;
  const T* Kg = Qg + hr;
  const T* Vg = Qg + 2 * hr;
  const T* dOg = reinterpret_cast<const T*>(a.dctx) + (int64_t)b * s * a.ld_ctx + hd * D;
  const int q0 = qb * BQ, q0w = q0 + wave * 32, my_q = q0w + l32;
  const float c = kLog2e * rsqrtf((float)D);
  const int64_t stat = ((int64_t)b * a.heads + hd) * s;
  const float lse_q = my_q < s ? a.lse[stat + my_q] * kLog2e : 0.f;
  const float delta_q = my_q < s ? a.delta[stat + my_q] : 0.f;

  Frag8<T> qf[D / 16], df[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_q < s) {
      load_frag(qf[st], Qg + (int64_t)my_q * a.ld_qkv + st * 16 + grp * 8);
      load_frag(df[st], dOg + (int64_t)my_q * a.ld_ctx + st * 16 + grp * 8);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      frag_from_f32(qf[st], z);
      frag_from_f32(df[st], z);
    }
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  const int kv_end = CAUSAL ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  KT k_ld, v_ld;
  TT kt_ld;
  k_ld.load(Kg, a.ld_qkv, 0, s, tid);
  v_ld.load(Vg, a.ld_qkv, 0, s, tid);
  kt_ld.load(Kg, a.ld_qkv, 0, s, tid);
  k_ld.store(sK[0], tid);
  v_ld.store(sV[0], tid);
  kt_ld.store(sKt[0], tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = NB == 1 ? 0 : t & 1, kv0 = t * BKV;
    const bool more = t + 1 < ntiles;
    if (more) {
      k_ld.load(Kg, a.ld_qkv, kv0 + BKV, s, tid);
      v_ld.load(Vg, a.ld_qkv, kv0 + BKV, s, tid);
      kt_ld.load(Kg, a.ld_qkv, kv0 + BKV, s, tid);
    }
    if (!CAUSAL || kv0 <= q0w + 31) {
      f32x16 sc[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[kt][r] = 0.f; dp[kt][r] = 0.f; }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          Frag8<T> kf, vf;
          load_frag(kf, &sK[cur][(kt * 32 + l32) * KT::kLd + st * 16 + grp * 8]);
          load_frag(vf, &sV[cur][(kt * 32 + l32) * KT::kLd + st * 16 + grp * 8]);
          mfma_step(sc[kt], kf, qf[st]);
          mfma_step(dp[kt], vf, df[st]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kt * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
          const bool ok = key < s && (!CAUSAL || key <= my_q) && my_q < s;
          const float p = ok ? exp2f(sc[kt][r] * c - lse_q) : 0.f;
          sc[kt][r] = p * (dp[kt][r] - delta_q);   // dS^T
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag8<T> sf;
        acc_frag(sf, sc[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          Frag8<T> kf;
          load_frag(kf, &sKt[cur][(dt * 32 + l32) * TT::kLd + ks * 16 + grp * 8]);
          mfma_step(dq[dt], kf, sf);
        }
      }
    }
    if (more) {
      if (NB == 1) __syncthreads();   // one buffer: every wave is past its reads of it
      k_ld.store(sK[NB == 1 ? 0 : cur ^ 1], tid);
      v_ld.store(sV[NB == 1 ? 0 : cur ^ 1], tid);
      kt_ld.store(sKt[NB == 1 ? 0 : cur ^ 1], tid);
    }
    __syncthreads();
  }
  if (my_q < s) {
    T* dQg = reinterpret_cast<T*>(a.dqkv) + (int64_t)b * s * a.ld_qkv + hd * D;
    store_rows<T, D>(dQg, a.ld_qkv, my_q, dq, rsqrtf((float)D), grp);
  }
}

// ------------------------------------------------------------------ backward: dK, dV
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(Args a) {
  constexpr int NT = 256, BKB = 128, BQ = 64;
  constexpr int NB = bwd_buffers<T, D>();
  using RT = RowTile<T, D, BQ, NT>;
  using TT = TransTile<T, D, NT>;
  __shared__ __attribute__((aligned(16))) T sQ[NB][BQ * RT::kLd];
  __shared__ __attribute__((aligned(16))) T sdO[NB][BQ * RT::kLd];
  __shared__ __attribute__((aligned(16))) T sQt[NB][D * TT::kLd];
  __shared__ __attribute__((aligned(16))) T sdOt[NB][D * TT::kLd];
  __shared__ __attribute__((aligned(16))) float sL[NB][BQ];
  __shared__ __attribute__((aligned(16))) float sDl[NB][BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, grp = lane >> 5;
  // 1-D grid dealt heaviest key tiles (the first ones, under a causal mask) first over all heads
  const int bhs = a.batch * a.heads, bh = blockIdx.x % bhs, kb = blockIdx.x / bhs;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int s = a.seq, hr = a.heads * D;
  const T* Qg = reinterpret_cast<const T*>(a.qkv) + (int64_t)b * s * a.ld_qkv + hd * D;
  const T* Kg = Qg + hr;
  const T* Vg = Qg + 2 * hr;
  const T* dOg = reinterpret_cast<const T*>(a.dctx) + (int64_t)b * s * a.ld_ctx + hd * D;
  const int64_t stat = ((int64_t)b * a.heads + hd) * s;
  const int k0 = kb * BKB, k0w = k0 + wave * 32, my_k = k0w + l32;
  const float c = kLog2e * rsqrtf((float)D);

  Frag8<T> kf[D / 16], vf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_k < s) {
      load_frag(kf[st], Kg + (int64_t)my_k * a.ld_qkv + st * 16 + grp * 8);
      load_frag(vf[st], Vg + (int64_t)my_k * a.ld_qkv + st * 16 + grp * 8);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      frag_from_f32(kf[st], z);
      frag_from_f32(vf[st], z);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[dt][r] = 0.f; dv[dt][r] = 0.f; }

  const int qs = CAUSAL ? (k0 / BQ) * BQ : 0;
  const int ntiles = s > qs ? (s - qs + BQ - 1) / BQ : 0;
  RT q_ld, d_ld;
  TT qt_ld, dt_ld;
  auto load_tile = [&](int q0) {
    q_ld.load(Qg, a.ld_qkv, q0, s, tid);
    d_ld.load(dOg, a.ld_ctx, q0, s, tid);
    qt_ld.load(Qg, a.ld_qkv, q0, s, tid);
    dt_ld.load(dOg, a.ld_ctx, q0, s, tid);
  };
  auto store_tile = [&](int buf, int q0) {
    q_ld.store(sQ[buf], tid);
    d_ld.store(sdO[buf], tid);
    qt_ld.store(sQt[buf], tid);
    dt_ld.store(sdOt[buf], tid);
    if (tid < BQ) {
      const int q = q0 + tid;
      sL[buf][tid] = q < s ? a.lse[stat + q] * kLog2e : 0.f;
      sDl[buf][tid] = q < s ? a.delta[stat + q] : 0.f;
    }
  };
  if (ntiles > 0) {
    load_tile(qs);
    store_tile(0, qs);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = NB == 1 ? 0 : t & 1, q0 = qs + t * BQ;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(q0 + BQ);
    if (!CAUSAL || q0 + BQ - 1 >= k0w) {
      f32x16 sc[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[qt][r] = 0.f; dp[qt][r] = 0.f; }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          Frag8<T> qf, df;
          load_frag(qf, &sQ[cur][(qt * 32 + l32) * RT::kLd + st * 16 + grp * 8]);
          load_frag(df, &sdO[cur][(qt * 32 + l32) * RT::kLd + st * 16 + grp * 8]);
          mfma_step(sc[qt], qf, kf[st]);   // S[q][key], lane owns key
          mfma_step(dp[qt], df, vf[st]);   // dP[q][key]
        }
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int qo = qt * 32 + 8 * rq + 4 * grp;
          const f32x4 lq = *reinterpret_cast<const f32x4*>(&sL[cur][qo]);
          const f32x4 dq = *reinterpret_cast<const f32x4*>(&sDl[cur][qo]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e, q = q0 + qo + e;
            const bool ok = q < s && my_k < s && (!CAUSAL || my_k <= q);
            const float p = ok ? exp2f(sc[qt][r] * c - lq[e]) : 0.f;
            sc[qt][r] = p;                          // P
            dp[qt][r] = p * (dp[qt][r] - dq[e]);    // dS
          }
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag8<T> pf, sf;
        acc_frag(pf, sc[ks >> 1], 8 * (ks & 1));
        acc_frag(sf, dp[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          Frag8<T> of, qf;
          load_frag(of, &sdOt[cur][(dt * 32 + l32) * TT::kLd + ks * 16 + grp * 8]);
          load_frag(qf, &sQt[cur][(dt * 32 + l32) * TT::kLd + ks * 16 + grp * 8]);
          mfma_step(dv[dt], of, pf);
          mfma_step(dk[dt], qf, sf);
        }
      }
    }
    if (more) {
      if (NB == 1) __syncthreads();   // one buffer: every wave is past its reads of it
      store_tile(NB == 1 ? 0 : cur ^ 1, q0 + BQ);
    }
    __syncthreads();
  }
  if (my_k < s) {
    T* dKg = reinterpret_cast<T*>(a.dqkv) + (int64_t)b * s * a.ld_qkv + hr + hd * D;
    store_rows<T, D>(dKg, a.ld_qkv, my_k, dk, rsqrtf((float)D), grp);
    store_rows<T, D>(dKg + hr, a.ld_qkv, my_k, dv, 1.f, grp);
  }
}

// ------------------------------------------------------------------ bf16 kernels
// bf16 version without register transposes. Every tile lives in LDS in its
// natural [row][d] layout; transposed MFMA operands (V^T, K^T, Q^T, dO^T) are
// read from it with ds_read_b64_tr_b16. To make the score accumulators come
// out with keys (or queries) in natural order in each lane's k-slots, the
// score MFMA's A operand takes tile row swap23(i) for accumulator row i (bits
// 2 and 3 of the row offset swapped): accumulator element r of lane group g
// then holds row 16*(r/8) + 8*g + r%8, which is exactly k-slot r%8 of the
// next MFMA's step r/8 -- the layout a transpose read of the natural tile
// delivers for the other operand.
//
// LDS rows are 8 (d=64) or 16 (d=96, 128; d=96 padded) 16-B chunks; chunk c
// of row r sits at c ^ swz_a(r) within its aligned group of 8. swz_a maps the
// rows read by any 8 consecutive lanes of a permuted row read
// ({0..3, 8..11} + 16k or {4..7, 12..15} + 16k) and any 4 consecutive rows of
// a transpose read to distinct 16-B bank groups.

__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
__device__ __forceinline__ int swz_a(int r) { return ((r & 3) << 1) | ((r >> 3) & 1); }

typedef short s16x4 __attribute__((__vector_size__(8)));

template <int D, int NT>
struct NatTile {
  static constexpr int kLC = D / 8;                  // 16-B chunks of data per row
  static constexpr int kRC = D == 64 ? 8 : 16;       // chunks per LDS row
  static constexpr int kRowBytes = kRC * 16;
  static constexpr int kBytes = 64 * kRowBytes;
  static constexpr int kTotal = 64 * kLC;
  static constexpr int kPer = (kTotal + NT - 1) / NT;
  static_assert(NT % 64 == 0, "whole waves per workgroup");
  u32x4 r[kPer];
  __device__ __forceinline__ static int phys(int row, int c) { return (c & ~7) | ((c ^ swz_a(row)) & 7); }
  // A thread's chunks of a tile, fixed over the loop: byte offset from the
  // tile's first row (row stride ld elements) and LDS byte offset; voff < 0
  // marks a slot past the tile.
  struct Map {
    int voff[kPer], loff[kPer];
  };
  __device__ __forceinline__ static Map map(int64_t ld, int tid) {
    Map m;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = tid + i * NT;
      const int row = p / kLC, c = p % kLC;
      m.voff[i] = p < kTotal ? (int)(((int64_t)row * ld + c * 8) * 2) : -1;
      m.loff[i] = row * kRowBytes + phys(row, c) * 16;
    }
    return m;
  }
  // rows [row0, row0+64) of a head's [rows][d] block at base (row stride ld),
  // through a buffer resource from row row0 that ends at the last valid
  // element of row nrows-1: rows past it read as 0
  __device__ __forceinline__ void load(const Map& m, const bf16* base, int64_t ld, int row0, int nrows) {
#if defined(__HIP_DEVICE_COMPILE__)   // the buffer-resource type exists only in the device pass
    const int64_t bytes = nrows > row0 ? ((int64_t)(nrows - 1 - row0) * ld + D) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base + (int64_t)row0 * ld), (short)0,
                                          bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (valid(m, i)) r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, m.voff[i], 0, 0);
#endif
  }
  __device__ __forceinline__ void store(const Map& m, char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (valid(m, i)) st16(lds + m.loff[i], r[i]);
  }
  // Slot i of a thread holds a chunk of the tile. kTotal is a multiple of 64
  // and every wave's slots start at a multiple of 64, so a slot is valid for
  // all lanes of a wave or for none: lane 0 decides (a scalar branch instead
  // of an exec mask around every load and store).
  __device__ __forceinline__ static bool valid(const Map& m, int i) {
    if constexpr (kTotal % NT == 0) return true;
    else return __builtin_amdgcn_readfirstlane(m.voff[i]) >= 0;
  }
  // 8 consecutive d-values (chunk c) of one row
  __device__ __forceinline__ static void row_frag(Frag8<bf16>& f, const char* lds, int row, int c) {
    load_frag(f, reinterpret_cast<const bf16*>(lds + row * kRowBytes + phys(row, c) * 16));
  }
  // transposed fragment: lane (column mn0 + lane%32, group g) gets rows k0 + 8g .. k0 + 8g + 7
  __device__ __forceinline__ static void tr_frag(Frag8<bf16>& f, const char* lds, int k0, int mn0, int lane) {
    const int G = lane >> 4, s = lane & 15, e = s >> 2, q = s & 3;
    const int mn = mn0 + 16 * (G & 1) + 4 * q;
    const int k = k0 + 8 * (G >> 1) + e;                 // swz_a(k) == swz_a(k + 4)
    const char* p0 = lds + k * kRowBytes + phys(k, mn >> 3) * 16 + (q & 1) * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0 + 4 * kRowBytes));
    __builtin_memcpy(reinterpret_cast<char*>(&f.v), &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&f.v) + 8, &hi, 8);
  }
};

// KW waves of 32 queries each per workgroup (BQ = 32 KW). SPL = 2 (used
// when the grid has under two waves per SIMD): a second group of KW waves
// takes every other key tile of the same queries; their partial (O, max,
// sum) are merged at the end through LDS in a fixed order. Forms: (KW 4,
// SPL 1) by default, (4, 2) for small grids at head size 64, (2, 2) at 96
// and 128 (one wave per SIMD there: twice the workgroups of half the rows).
template <int D, bool CAUSAL, int SPL, int KW>
__global__ __launch_bounds__(64 * KW * SPL) __attribute__((amdgpu_waves_per_eu(KW * SPL == 8 ? 2 : (D == 64 ? 3 : 1)))) void attn_fwd_bf16_kernel(Args a) {
  constexpr int NT = 64 * KW * SPL, BQ = 32 * KW, BKV = 64;
  constexpr int kLanes = 64 * KW;   // lanes of one parity group
  using Tile = NatTile<D, NT>;
  __shared__ __attribute__((aligned(16))) char sK[2][SPL][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char sV[2][SPL][Tile::kBytes];
  __shared__ float sML[SPL == 2 ? 2 * kLanes : 1];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, grp = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave-level branches stay scalar
  const int wave = wid % KW, par = wid / KW;                    // query sub-tile, key-tile parity
  // 1-D grid dealt heaviest query tiles first over all heads (causal tiles
  // differ up to seq/BQ-fold in work, so the last to start are the short ones)
  const int bhs = a.batch * a.heads, bh = blockIdx.x % bhs;
  const int qb = gridDim.x / bhs - 1 - blockIdx.x / bhs;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int s = a.seq, hr = a.heads * D;
  const bf16* Qg = reinterpret_cast<const bf16*>(a.qkv) + (int64_t)b * s * a.ld_qkv + hd * D;
  const bf16* Kg = Qg + hr;
  const bf16* Vg = Qg + 2 * hr;
  const int q0 = qb * BQ, q0w = q0 + wave * 32, my_q = q0w + l32;
  const float c = kLog2e * rsqrtf((float)D);
  const int krow = swap23(l32);

  Frag8<bf16> qf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_q < s) load_frag(qf[st], Qg + (int64_t)my_q * a.ld_qkv + st * 16 + grp * 8);
    else { float z[8] = {0, 0, 0, 0, 0, 0, 0, 0}; frag_from_f32(qf[st], z); }
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;   // running max of raw scores, running sum

  const int kv_end = CAUSAL ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const int nsteps = (ntiles + SPL - 1) / SPL;   // SPL key tiles per step, one per parity
  Tile kl[SPL], vl[SPL];
  const typename Tile::Map mp = Tile::map(a.ld_qkv, tid);
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    kl[u].load(mp, Kg, a.ld_qkv, u * BKV, s);
    vl[u].load(mp, Vg, a.ld_qkv, u * BKV, s);
    kl[u].store(mp, sK[0][u]);
    vl[u].store(mp, sV[0][u]);
  }
  __syncthreads();

  for (int t = 0; t < nsteps; ++t) {
    const int cur = t & 1, kv0 = (t * SPL + par) * BKV;
    const bool more = t + 1 < nsteps;
    if (more) {
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        kl[u].load(mp, Kg, a.ld_qkv, ((t + 1) * SPL + u) * BKV, s);
        vl[u].load(mp, Vg, a.ld_qkv, ((t + 1) * SPL + u) * BKV, s);
      }
    }
    if (kv0 < kv_end && (!CAUSAL || kv0 <= q0w + 31)) {
      const char* tK = sK[cur][par];
      const char* tV = sV[cur][par];
      f32x16 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          Frag8<bf16> kf;
          Tile::row_frag(kf, tK, kt * 32 + krow, 2 * st + grp);
          mfma_step(sc[kt], kf, qf[st]);
        }
      }
      // key of accumulator element r of tile kt: kv0 + 32kt + 16(r/8) + 8grp + r%8
      if ((CAUSAL && kv0 + BKV - 1 > q0w) || kv0 + BKV > s) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kt + 16 * (r >> 3) + 8 * grp + (r & 7);
            if (key >= s || (CAUSAL && key > my_q)) sc[kt][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      // The reference max m moves only when some row's max has grown past it
      // by more than 2^kLazy in the exp2 domain (or on the first visible
      // tile): softmax does not depend on the reference, the probabilities
      // stay below 2^kLazy, and the rescale of O (D/2 multiplies per lane)
      // is skipped on most tiles of a long row.
      if (__any(mx != -INFINITY && (m == -INFINITY || (mx - m) * c > kLazy))) {
        const float m_new = fmaxf(m, mx);
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m = m_new;
      }
      const float mc = m == -INFINITY ? 0.f : m * c;
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[kt][r], c, -mc));
          sc[kt][r] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 32, kWave);
      l += sum;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag8<bf16> pf;
        acc_frag(pf, sc[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          Frag8<bf16> vf;
          Tile::tr_frag(vf, tV, ks * 16, dt * 32, lane);
          mfma_step(o[dt], vf, pf);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        kl[u].store(mp, sK[cur ^ 1][u]);
        vl[u].store(mp, sV[cur ^ 1][u]);
      }
    }
    __syncthreads();
  }

  if constexpr (SPL == 2) {
    // the odd-parity wave of each query sub-tile hands (O, max, sum) to its
    // partner through the free K stages: element e of lane i at [e][i]
    static_assert(D / 2 * kLanes * 4 <= (int)sizeof(sK), "the K stages must hold the exchanged O");
    float* xo = reinterpret_cast<float*>(&sK[0][0][0]);
    const int slot = wave * 64 + lane;
    if (par == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * kLanes + slot] = o[dt][r];
      sML[slot] = m;
      sML[kLanes + slot] = l;
    }
    __syncthreads();
    if (par == 1) return;
    const float m1 = sML[slot], l1 = sML[kLanes + slot];
    const float mn = fmaxf(m, m1);
    const float mc = mn == -INFINITY ? 0.f : mn * c;
    const float a0 = __builtin_amdgcn_exp2f(m * c - mc), a1 = __builtin_amdgcn_exp2f(m1 * c - mc);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * a0 + xo[(dt * 16 + r) * kLanes + slot] * a1;
    l = l * a0 + l1 * a1;
    m = mn;
  }

  if (my_q < s) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* Og = reinterpret_cast<bf16*>(a.ctx) + (int64_t)b * s * a.ld_ctx + hd * D;
    store_rows<bf16, D>(Og, a.ld_ctx, my_q, o, inv, grp);
    if (grp == 0) a.lse[((int64_t)b * a.heads + hd) * s + my_q] = (m * c) * kLn2 + logf(l);
  }
}

// KW waves of 32 queries per workgroup; SPL = 2: a second group of KW waves
// takes every other key tile; the two partial dQ are added at the end (even
// parity first). Forms as for the forward.
template <int D, int SPL, int KW>
struct DqLds {
  using Tile = NatTile<D, 64 * KW * SPL>;
  char sK[2][SPL][Tile::kBytes];
  char sV[2][SPL][Tile::kBytes];
};
// The dQ kernel's work for query tile blk of a grid of nblk (heaviest first).
template <int D, bool CAUSAL, int SPL, int KW>
__device__ __forceinline__ void attn_bwd_dq_bf16_body(const Args& a, DqLds<D, SPL, KW>& L, int blk, int nblk) {
  constexpr int NT = 64 * KW * SPL, BQ = 32 * KW, BKV = 64;
  constexpr int kLanes = 64 * KW;   // lanes of one parity group
  using Tile = NatTile<D, NT>;
  auto& sK = L.sK;
  auto& sV = L.sV;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, grp = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave-level branches stay scalar
  const int wave = wid % KW, par = wid / KW;                    // query sub-tile, key-tile parity
  // 1-D grid dealt heaviest query tiles first over all heads (causal tiles
  // differ up to seq/BQ-fold in work, so the last to start are the short ones)
  const int bhs = a.batch * a.heads, bh = blk % bhs;
  const int qb = nblk / bhs - 1 - blk / bhs;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int s = a.seq, hr = a.heads * D;
  const bf16* Qg = reinterpret_cast<const bf16*>(a.qkv) + (int64_t)b * s * a.ld_qkv + hd * D;
  const bf16* Kg = Qg + hr;
  const bf16* Vg = Qg + 2 * hr;
  const bf16* dOg = reinterpret_cast<const bf16*>(a.dctx) + (int64_t)b * s * a.ld_ctx + hd * D;
  const int q0 = qb * BQ, q0w = q0 + wave * 32, my_q = q0w + l32;
  const float c = kLog2e * rsqrtf((float)D);
  const int64_t stat = ((int64_t)b * a.heads + hd) * s;
  const float lse_q = my_q < s ? a.lse[stat + my_q] * kLog2e : 0.f;
  const float delta_q = my_q < s ? a.delta[stat + my_q] : 0.f;
  const int krow = swap23(l32);

  Frag8<bf16> qf[D / 16], df[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_q < s) {
      load_frag(qf[st], Qg + (int64_t)my_q * a.ld_qkv + st * 16 + grp * 8);
      load_frag(df[st], dOg + (int64_t)my_q * a.ld_ctx + st * 16 + grp * 8);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      frag_from_f32(qf[st], z);
      frag_from_f32(df[st], z);
    }
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  const int kv_end = CAUSAL ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const int nsteps = (ntiles + SPL - 1) / SPL;   // SPL key tiles per step, one per parity
  Tile kl[SPL], vl[SPL];
  const typename Tile::Map mp = Tile::map(a.ld_qkv, tid);
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    kl[u].load(mp, Kg, a.ld_qkv, u * BKV, s);
    vl[u].load(mp, Vg, a.ld_qkv, u * BKV, s);
    kl[u].store(mp, sK[0][u]);
    vl[u].store(mp, sV[0][u]);
  }
  __syncthreads();

  for (int t = 0; t < nsteps; ++t) {
    const int cur = t & 1, kv0 = (t * SPL + par) * BKV;
    const bool more = t + 1 < nsteps;
    if (more) {
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        kl[u].load(mp, Kg, a.ld_qkv, ((t + 1) * SPL + u) * BKV, s);
        vl[u].load(mp, Vg, a.ld_qkv, ((t + 1) * SPL + u) * BKV, s);
      }
    }
    if (kv0 < kv_end && (!CAUSAL || kv0 <= q0w + 31)) {
      const char* tK = sK[cur][par];
      const char* tV = sV[cur][par];
      // wave-uniform (q0w comes from the wave index): one scalar branch skips the
      // masking of every score on tiles that need none (a per-lane flag would
      // run the masking code under an exec mask for every score of every tile)
      const bool mask = (CAUSAL && kv0 + BKV - 1 > q0w) || kv0 + BKV > s || q0w + 32 > s;
      // the tile's two 32-key halves one after the other (half the score
      // registers live at a time, so the accumulators stay in VGPRs)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 sc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          Frag8<bf16> kf, vf;
          Tile::row_frag(kf, tK, kt * 32 + krow, 2 * st + grp);
          Tile::row_frag(vf, tV, kt * 32 + krow, 2 * st + grp);
          mfma_step(sc, kf, qf[st]);
          mfma_step(dp, vf, df[st]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -lse_q));
        if (mask) {   // one scalar branch around the masking of the whole tile
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kt + 16 * (r >> 3) + 8 * grp + (r & 7);
            if (key >= s || (CAUSAL && key > my_q) || my_q >= s) sc[r] = 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = sc[r] * (dp[r] - delta_q);   // dS^T
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int ks = 2 * kt + kh;
          Frag8<bf16> sf;
          acc_frag(sf, sc, 8 * kh);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            Frag8<bf16> kf;
            Tile::tr_frag(kf, tK, ks * 16, dt * 32, lane);
            mfma_step(dq[dt], kf, sf);
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        kl[u].store(mp, sK[cur ^ 1][u]);
        vl[u].store(mp, sV[cur ^ 1][u]);
      }
    }
    __syncthreads();
  }
  if constexpr (SPL == 2) {
    // odd-parity partial dQ through the free K stages: element e of lane i at [e][i]
    static_assert(D / 2 * kLanes * 4 <= (int)sizeof(sK), "the K stages must hold the exchanged dQ");
    float* xq = reinterpret_cast<float*>(&sK[0][0][0]);
    const int slot = wave * 64 + lane;
    if (par == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xq[(dt * 16 + r) * kLanes + slot] = dq[dt][r];
    }
    __syncthreads();
    if (par == 1) return;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[dt][r] += xq[(dt * 16 + r) * kLanes + slot];
  }
  if (my_q < s) {
    bf16* dQg = reinterpret_cast<bf16*>(a.dqkv) + (int64_t)b * s * a.ld_qkv + hd * D;
    store_rows<bf16, D>(dQg, a.ld_qkv, my_q, dq, rsqrtf((float)D), grp);
  }
}
template <int D, bool CAUSAL, int SPL, int KW>
__global__ __launch_bounds__(64 * KW * SPL) __attribute__((amdgpu_waves_per_eu(KW * SPL == 8 ? 2 : (D == 64 ? 3 : 1)))) void attn_bwd_dq_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) DqLds<D, SPL, KW> L;
  attn_bwd_dq_bf16_body<D, CAUSAL, SPL, KW>(a, L, (int)blockIdx.x, (int)gridDim.x);
}

// KW waves of 32 keys each per workgroup (BKB = 32 KW keys). SPL = 2: a
// second group of KW waves takes every other query tile; the two partial dK
// and dV are added at the end (even parity first). Forms: (KW 4, SPL 1) by
// default; (4, 2) for small grids at head size 64; (2, 2) for small grids at
// 96 and 128, where two waves per SIMD would not fit the registers: twice the
// workgroups of half the keys, one wave per SIMD.
template <int D, int SPL, int KW>
struct DkdvLds {
  using Tile = NatTile<D, 64 * KW * SPL>;
  char sQ[2][SPL][Tile::kBytes];
  char sdO[2][SPL][Tile::kBytes];
  float sL[2][SPL][64];
  float sDl[2][SPL][64];
};
// The dK/dV kernel's work for key tile blk of a grid of nblk (heaviest first).
template <int D, bool CAUSAL, int SPL, int KW>
__device__ __forceinline__ void attn_bwd_dkdv_bf16_body(const Args& a, DkdvLds<D, SPL, KW>& L, int blk, int nblk) {
  constexpr int NT = 64 * KW * SPL, BKB = 32 * KW, BQ = 64;
  using Tile = NatTile<D, NT>;
  auto& sQ = L.sQ;
  auto& sdO = L.sdO;
  auto& sL = L.sL;
  auto& sDl = L.sDl;
  (void)nblk;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, grp = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave-level branches stay scalar
  const int wave = wid % KW, par = wid / KW;                    // key sub-tile, query-tile parity
  // 1-D grid dealt heaviest key tiles (the first ones, under a causal mask) first over all heads
  const int bhs = a.batch * a.heads, bh = blk % bhs, kb = blk / bhs;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int s = a.seq, hr = a.heads * D;
  const bf16* Qg = reinterpret_cast<const bf16*>(a.qkv) + (int64_t)b * s * a.ld_qkv + hd * D;
  const bf16* Kg = Qg + hr;
  const bf16* Vg = Qg + 2 * hr;
  const bf16* dOg = reinterpret_cast<const bf16*>(a.dctx) + (int64_t)b * s * a.ld_ctx + hd * D;
  const int64_t stat = ((int64_t)b * a.heads + hd) * s;
  const int k0 = kb * BKB, k0w = k0 + wave * 32, my_k = k0w + l32;
  const float c = kLog2e * rsqrtf((float)D);
  const int qrow = swap23(l32);

  Frag8<bf16> kf[D / 16], vf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_k < s) {
      load_frag(kf[st], Kg + (int64_t)my_k * a.ld_qkv + st * 16 + grp * 8);
      load_frag(vf[st], Vg + (int64_t)my_k * a.ld_qkv + st * 16 + grp * 8);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      frag_from_f32(kf[st], z);
      frag_from_f32(vf[st], z);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[dt][r] = 0.f; dv[dt][r] = 0.f; }

  const int qs = CAUSAL ? (k0 / BQ) * BQ : 0;
  const int ntiles = s > qs ? (s - qs + BQ - 1) / BQ : 0;
  const int nsteps = (ntiles + SPL - 1) / SPL;   // SPL query tiles per step, one per parity
  Tile ql[SPL], dl[SPL];
  // statistics of the SPL query tiles from q0 (rows past the sequence read 0)
  auto stage_stats = [&](int buf, int q0) {
    if (tid < BQ * SPL) {
      const int u = tid / BQ, j = tid % BQ, q = q0 + u * BQ + j;
      sL[buf][u][j] = q < s ? a.lse[stat + q] * kLog2e : 0.f;
      sDl[buf][u][j] = q < s ? a.delta[stat + q] : 0.f;
    }
  };
  const typename Tile::Map mq = Tile::map(a.ld_qkv, tid), md = Tile::map(a.ld_ctx, tid);
  if (ntiles > 0) {
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      ql[u].load(mq, Qg, a.ld_qkv, qs + u * BQ, s);
      dl[u].load(md, dOg, a.ld_ctx, qs + u * BQ, s);
      ql[u].store(mq, sQ[0][u]);
      dl[u].store(md, sdO[0][u]);
    }
    stage_stats(0, qs);
  }
  __syncthreads();

  for (int t = 0; t < nsteps; ++t) {
    const int cur = t & 1, q0 = qs + (t * SPL + par) * BQ;
    const bool more = t + 1 < nsteps;
    if (more) {
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        ql[u].load(mq, Qg, a.ld_qkv, qs + ((t + 1) * SPL + u) * BQ, s);
        dl[u].load(md, dOg, a.ld_ctx, qs + ((t + 1) * SPL + u) * BQ, s);
      }
    }
    if (q0 < s && (!CAUSAL || q0 + BQ - 1 >= k0w)) {
      const char* tQ = sQ[cur][par];
      const char* tdO = sdO[cur][par];
      const float* tL = sL[cur][par];
      const float* tDl = sDl[cur][par];
      // wave-uniform, as in the dQ kernel
      const bool mask = (CAUSAL && q0 < k0w + 31) || q0 + BQ > s || k0w + 32 > s;
      // the tile's two 32-query halves one after the other (half the score
      // registers live at a time)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x16 sc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          Frag8<bf16> qf, df;
          Tile::row_frag(qf, tQ, qt * 32 + qrow, 2 * st + grp);
          Tile::row_frag(df, tdO, qt * 32 + qrow, 2 * st + grp);
          mfma_step(sc, qf, kf[st]);   // S[q][key], lane owns key
          mfma_step(dp, df, vf[st]);   // dP[q][key]
        }
        // query of accumulator element r: q0 + 32qt + 16(r/8) + 8grp + r%8
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int qo = qt * 32 + 16 * (rq >> 1) + 8 * grp + 4 * (rq & 1);
          const f32x4 lq = *reinterpret_cast<const f32x4*>(&tL[qo]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * rq + e] = __builtin_amdgcn_exp2f(fmaf(sc[4 * rq + e], c, -lq[e]));
        }
        // masking in one pass behind one scalar branch (the per-element form
        // left a branch around every score)
        if (mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = q0 + qt * 32 + 16 * (r >> 3) + 8 * grp + (r & 7);
            if (q >= s || my_k >= s || (CAUSAL && my_k > q)) sc[r] = 0.f;
          }
        }
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int qo = qt * 32 + 16 * (rq >> 1) + 8 * grp + 4 * (rq & 1);
          const f32x4 dq = *reinterpret_cast<const f32x4*>(&tDl[qo]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * rq + e] = sc[4 * rq + e] * (dp[4 * rq + e] - dq[e]);   // dS
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int ks = 2 * qt + kh;
          Frag8<bf16> pf, sf;
          acc_frag(pf, sc, 8 * kh);
          acc_frag(sf, dp, 8 * kh);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            Frag8<bf16> of, qf;
            Tile::tr_frag(of, tdO, ks * 16, dt * 32, lane);
            Tile::tr_frag(qf, tQ, ks * 16, dt * 32, lane);
            mfma_step(dv[dt], of, pf);
            mfma_step(dk[dt], qf, sf);
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        ql[u].store(mq, sQ[cur ^ 1][u]);
        dl[u].store(md, sdO[cur ^ 1][u]);
      }
      stage_stats(cur ^ 1, qs + (t + 1) * SPL * BQ);
    }
    __syncthreads();
  }
  if constexpr (SPL == 2) {
    // odd-parity partial dK (through the free Q stages) and dV (through the
    // dO stages): element e of lane i at [e][i]
    constexpr int kLanes = 64 * KW;   // lanes of one parity group
    static_assert(D / 2 * kLanes * 4 <= (int)sizeof(sQ), "the Q stages must hold the exchanged dK");
    float* xk = reinterpret_cast<float*>(&sQ[0][0][0]);
    float* xv = reinterpret_cast<float*>(&sdO[0][0][0]);
    const int slot = wave * 64 + lane;
    if (par == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xk[(dt * 16 + r) * kLanes + slot] = dk[dt][r];
          xv[(dt * 16 + r) * kLanes + slot] = dv[dt][r];
        }
    }
    __syncthreads();
    if (par == 1) return;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[dt][r] += xk[(dt * 16 + r) * kLanes + slot];
        dv[dt][r] += xv[(dt * 16 + r) * kLanes + slot];
      }
  }
  if (my_k < s) {
    bf16* dKg = reinterpret_cast<bf16*>(a.dqkv) + (int64_t)b * s * a.ld_qkv + hr + hd * D;
    store_rows<bf16, D>(dKg, a.ld_qkv, my_k, dk, rsqrtf((float)D), grp);
    store_rows<bf16, D>(dKg + hr, a.ld_qkv, my_k, dv, 1.f, grp);
  }
}
template <int D, bool CAUSAL, int SPL, int KW>
__global__ __launch_bounds__(64 * KW * SPL) __attribute__((amdgpu_waves_per_eu(KW * SPL == 8 ? 2 : (D == 64 ? 2 : 1)))) void attn_bwd_dkdv_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) DkdvLds<D, SPL, KW> L;
  attn_bwd_dkdv_bf16_body<D, CAUSAL, SPL, KW>(a, L, (int)blockIdx.x, (int)gridDim.x);
}

// dK/dV and dQ as the two roles of one grid (small grids): the two kernels
// are independent (both read Q, K, V, dO and the row statistics; they write
// dK/dV and dQ), and under a causal mask each leaves most CUs idle while its
// heaviest tiles run. Workgroups alternate dK/dV, dQ in each role's own
// heaviest-first order (the longer role's surplus last), so the light tiles of
// one fill the CUs the other's heavy tiles leave; one LDS allocation serves
// either role.
template <int D, int SPL, int KW>
union AttnBwdLds {
  DkdvLds<D, SPL, KW> kv;
  DqLds<D, SPL, KW> q;
};
template <int D, bool CAUSAL, int SPL, int KW>
__global__ __launch_bounds__(64 * KW * SPL) __attribute__((amdgpu_waves_per_eu(KW * SPL == 8 ? 2 : 1))) void attn_bwd_pair_kernel(Args a, int n_kv, int n_q) {
  __shared__ __attribute__((aligned(16))) AttnBwdLds<D, SPL, KW> L;
  const int blk = (int)blockIdx.x, m = n_kv < n_q ? n_kv : n_q;
  if (blk < 2 * m) {
    if ((blk & 1) == 0) attn_bwd_dkdv_bf16_body<D, CAUSAL, SPL, KW>(a, L.kv, blk >> 1, n_kv);
    else attn_bwd_dq_bf16_body<D, CAUSAL, SPL, KW>(a, L.q, blk >> 1, n_q);
  } else if (n_kv > n_q) {
    attn_bwd_dkdv_bf16_body<D, CAUSAL, SPL, KW>(a, L.kv, blk - m, n_kv);
  } else {
    attn_bwd_dq_bf16_body<D, CAUSAL, SPL, KW>(a, L.q, blk - m, n_q);
  }
}

// Visible query-key pairs over all heads and sequences (causal: s(s+1)/2 each).
double attn_pairs(const AttnDesc& d) {
  const double s = d.seq;
  return (double)d.batch * d.heads * (d.causal ? s * (s + 1) / 2 : s * s);
}

// The eight-wave form (tiles of the looped axis dealt over two wave groups)
// when the four-wave grid would leave fewer than two waves per SIMD of the
// chip: each workgroup of 128 rows then has twice the waves in flight.
bool attn_split(const AttnDesc& d) {
  if (const char* f = getenv("TPL_ATTN_SPLIT")) return atoi(f) != 0;
  const int64_t waves = (int64_t)((d.seq + 127) / 128) * d.batch * d.heads * 4;
  return waves < 2 * 4 * (int64_t)device_cu_count();
}

// dK/dV and dQ in one launch (attn_bwd_pair_kernel) when each role's n
// workgroups fit one round; TPL_ATTN_BWD_PAIR=0/1 forces the choice (tests).
bool attn_bwd_paired(int64_t n) {
  if (const char* f = getenv("TPL_ATTN_BWD_PAIR")) return atoi(f) != 0;
  return n <= (int64_t)device_cu_count();
}

Args make_args(const AttnDesc& d) {
  Args a;
  a.qkv = static_cast<const char*>(d.qkv); a.ld_qkv = d.ld_qkv;
  a.ctx = static_cast<char*>(d.ctx); a.ld_ctx = d.ld_ctx;
  a.lse = d.lse;
  a.dctx = static_cast<const char*>(d.dctx);
  a.dqkv = static_cast<char*>(d.dqkv);
  a.delta = d.delta;
  a.batch = d.batch; a.heads = d.heads; a.seq = d.seq;
  return a;
}

template <typename T, int D>
hipError_t fwd_t(const AttnDesc& d, hipStream_t s) {
  Args a = make_args(d);
  dim3 grid((unsigned)(((d.seq + 127) / 128) * d.batch * d.heads));
  if constexpr (sizeof(T) == 2) {
    if (attn_split(d)) {   // small grids: see attn_fwd_bf16_kernel (64 rows per workgroup measured
      constexpr int kKw = D >= 96 ? 2 : 4;    // faster at head sizes 96 and 128: 8.3B rank 28 -> 21 us)
      dim3 g2((unsigned)(((d.seq + 32 * kKw - 1) / (32 * kKw)) * d.batch * d.heads));
      if (d.causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, 2, kKw>), g2, dim3(128 * kKw), 0, s, a);
      else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, 2, kKw>), g2, dim3(128 * kKw), 0, s, a);
    } else {
      if (d.causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, 1, 4>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, 1, 4>), grid, dim3(256), 0, s, a);
    }
  } else {
    if (d.causal) hipLaunchKernelGGL((attn_fwd_kernel<T, D, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<T, D, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_t(const AttnDesc& d, hipStream_t s) {
  Args a = make_args(d);
  {
    TraceScope trace(K_ATTN_BWD_PRE, s, (double)d.batch * d.seq * d.heads * d.head_dim * 2 * dtype_size(d.dtype));
    constexpr int kChunks = D * (int)sizeof(T) / 16;
    constexpr int G = kChunks <= 8 ? 8 : (kChunks <= 16 ? 16 : 32);
    const int64_t lanes = (int64_t)d.batch * d.heads * d.seq * G;
    hipLaunchKernelGGL((attn_bwd_pre_kernel<T, D>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(((d.seq + 127) / 128) * d.batch * d.heads));
  if constexpr (sizeof(T) == 2) {
    // small grids whose dK/dV and dQ workgroups each fit one round on the
    // CUs (one workgroup per CU: their LDS stages take over 64 KB): both as
    // two roles of one launch (8.3B rank 54.6 -> 42.5 us; with 1.5 rounds
    // each, as on the 175B rank, level, so those keep two launches)
    constexpr int kKw = D == 64 ? 4 : 2;   // the small-grid forms of both kernels
    const int64_t n = (int64_t)((d.seq + 32 * kKw - 1) / (32 * kKw)) * d.batch * d.heads;
    if (attn_split(d) && attn_bwd_paired(n)) {
      TraceScope trace(K_ATTN_BWD_PAIR, s, 8.0 * attn_pairs(d) * d.head_dim);   // dV, dP, dK; dQ's dP and dQ
      const dim3 g((unsigned)(2 * n));
      if (d.causal) hipLaunchKernelGGL((attn_bwd_pair_kernel<D, true, 2, kKw>), g, dim3(128 * kKw), 0, s, a, (int)n, (int)n);
      else hipLaunchKernelGGL((attn_bwd_pair_kernel<D, false, 2, kKw>), g, dim3(128 * kKw), 0, s, a, (int)n, (int)n);
      return hipGetLastError();
    }
  }
  {
    TraceScope trace(K_ATTN_BWD_DKDV, s, 6.0 * attn_pairs(d) * d.head_dim);   // dV, dP, dK
    if constexpr (sizeof(T) == 2) {
      // small grids: eight waves per 128 keys at head size 64; at 96 and 128
      // (where the dK, dV, K and V registers of two waves per SIMD would
      // spill) four waves per 64 keys, so twice the workgroups
      if (attn_split(d)) {
        constexpr int kKw = D == 64 ? 4 : 2;
        dim3 g2((unsigned)(((d.seq + 32 * kKw - 1) / (32 * kKw)) * d.batch * d.heads));
        if (d.causal) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, 2, kKw>), g2, dim3(128 * kKw), 0, s, a);
        else hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, false, 2, kKw>), g2, dim3(128 * kKw), 0, s, a);
      } else {
        if (d.causal) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, 1, 4>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, false, 1, 4>), grid, dim3(256), 0, s, a);
      }
    } else {
      if (d.causal) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, false>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TraceScope trace(K_ATTN_BWD_DQ, s, 2.0 * attn_pairs(d) * d.head_dim);     // dQ
  if constexpr (sizeof(T) == 2) {
    if (attn_split(d)) {   // small grids: see attn_bwd_dq_bf16_kernel (64 rows per workgroup
      constexpr int kKw = D >= 96 ? 2 : 4;    // measured faster at 96 and 128: 8.3B rank 30 -> 22 us)
      dim3 g2((unsigned)(((d.seq + 32 * kKw - 1) / (32 * kKw)) * d.batch * d.heads));
      if (d.causal) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, 2, kKw>), g2, dim3(128 * kKw), 0, s, a);
      else hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, false, 2, kKw>), g2, dim3(128 * kKw), 0, s, a);
    } else {
      if (d.causal) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, 1, 4>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, false, 1, 4>), grid, dim3(256), 0, s, a);
    }
  } else {
    if (d.causal) hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

// Head sizes 64, 96 and 128 in both storage types.
hipError_t launch_attn_fwd(const AttnDesc& d, hipStream_t s) {
  TraceScope trace(K_ATTN_FWD, s, 4.0 * attn_pairs(d) * d.head_dim);       // QK^T, PV
  if (d.dtype == DT_F32) {
    switch (d.head_dim) {
      case 64: return fwd_t<float, 64>(d, s);
      case 96: return fwd_t<float, 96>(d, s);
      case 128: return fwd_t<float, 128>(d, s);
    }
    return hipErrorInvalidValue;
  }
  switch (d.head_dim) {
    case 64: return fwd_t<bf16, 64>(d, s);
    case 96: return fwd_t<bf16, 96>(d, s);
    case 128: return fwd_t<bf16, 128>(d, s);
  }
  return hipErrorInvalidValue;
}
hipError_t launch_attn_bwd(const AttnDesc& d, hipStream_t s) {
  if (d.dtype == DT_F32) {
    switch (d.head_dim) {
      case 64: return bwd_t<float, 64>(d, s);
      case 96: return bwd_t<float, 96>(d, s);
      case 128: return bwd_t<float, 128>(d, s);
    }
    return hipErrorInvalidValue;
  }
  switch (d.head_dim) {
    case 64: return bwd_t<bf16, 64>(d, s);
    case 96: return bwd_t<bf16, 96>(d, s);
    case 128: return bwd_t<bf16, 128>(d, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpl
