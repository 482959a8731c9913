// Dense products of the parallel linear layers on gfx950 MFMA.
//
// Every contraction of the layer shard is C[M][N] = sum_k A(m,k) B(n,k):
//   forward  (NT): A = activations [M][K], B = weight [N][K]      (both K-major)
//   dgrad    (NN): A = dY [M][K'],         B = weight [K'][N]     (B N-major)
//   wgrad    (TN): A = dY^T via dY [K][M], B = X via [K][N]       (both MN-major)
// (guide page section 1.2: tensor parallelism splits one matrix product over
// devices; each rank runs its slice through this kernel.)
//
// Design:
//  * workgroup tile BM x BN, K-tile of 128 bytes per row (64 bf16 / 32 fp32),
//    two LDS buffers (one barrier per K-tile), the next K-tile prefetched into
//    registers while MFMAs consume the current one;
//  * LDS rows are 128 B = 8 chunks of 16 B, chunk c of row r stored at
//    c ^ ((r ^ r>>3) & 7) so that fragment reads (32 consecutive rows, one
//    chunk) and transposed writes (rows 8 apart) are bank-conflict free;
//  * MN-major operands are loaded as 8 k-rows x 16 B, transposed in registers
//    and written K-contiguous, so the MFMA loop is identical for all layouts;
//  * the wave tile is a grid of 32x32 outputs, each a v_mfma_f32_32x32x16_bf16
//    per 16 k (fp32: 8 x v_mfma_f32_32x32x2f32). The weight-side fragment is
//    the MFMA's A operand, so lane l owns output row m = l%32 and four
//    consecutive columns per accumulator quad: epilogue stores are 8/16 B;
//  * workgroups are renumbered so that consecutive tiles share an XCD (the
//    dispatcher deals workgroups to the 8 XCDs round-robin, each with its own
//    L2), then walked in groups of GROUP_M tile-rows for L2 reuse of B.
#include "common.h"
#include "kernels.h"

namespace tpl {

namespace {

constexpr int kRowBytes = 128;   // one LDS row = one K-tile of one output row/col
constexpr int kGroupM = 8;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

struct Args {
  const char* A; int64_t lda;
  const char* B; int64_t ldb;
  char* C; int64_t ldc;
  char* C2; int64_t ldc2;
  const char* bias;
  int M, N, K;
  int tiles_m, tiles_n;
};

// Load a K-major operand tile (ROWS x BK) to registers: ROWS*8 chunks of 16 B.
template <typename T, int ROWS, int NT>
struct KMajorLoader {
  static constexpr int kVec = 16 / sizeof(T);
  static constexpr int kLoads = ROWS * 8 / NT;
  static_assert(ROWS * 8 % NT == 0, "tile/threads mismatch");
  u32x4 r[kLoads];
  __device__ __forceinline__ void load(const char* base, int64_t ld, int row0, int rows_max, int k0,
                                       int kmax, int tid) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int idx = tid + i * NT;
      int row = idx >> 3, ch = idx & 7;
      int grow = row0 + row, gk = k0 + ch * kVec;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (grow < rows_max && gk < kmax) v = ld16(base + ((int64_t)grow * ld + gk) * sizeof(T));
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int idx = tid + i * NT;
      int row = idx >> 3, ch = idx & 7;
      st16(lds + row * kRowBytes + ((ch ^ swz(row)) << 4), r[i]);
    }
  }
};

// Load an MN-major operand tile: global [K][ld] with MN contiguous. Unit =
// 8 k-rows x one 16 B vector along MN; stored transposed (K-contiguous).
template <typename T, int ROWS, int NT>
struct MNMajorLoader {
  static constexpr int kVec = 16 / sizeof(T);
  static constexpr int kBK = kRowBytes / sizeof(T);
  static constexpr int kUnits = (kBK / 8) * (ROWS / kVec);
  static constexpr int kPer = (kUnits + NT - 1) / NT;
  u32x4 r[kPer][8];
  __device__ __forceinline__ void load(const char* base, int64_t ld, int mn0, int mn_max, int k0,
                                       int kmax, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      int mv = unit % (ROWS / kVec), kg = unit / (ROWS / kVec);
      int gmn = mn0 + mv * kVec;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int gk = k0 + kg * 8 + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (unit < kUnits && gk < kmax && gmn < mn_max)
          v = ld16(base + ((int64_t)gk * ld + gmn) * sizeof(T));
        r[u][j] = v;
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      if (unit >= kUnits) break;
      int mv = unit % (ROWS / kVec), kg = unit / (ROWS / kVec);
      if constexpr (sizeof(T) == 2) {
        // 8x8 transpose of 16-bit values: out row c, k pair p = (in[2p][c], in[2p+1][c]).
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          u32x4 o;
#pragma unroll
          for (int p = 0; p < 4; ++p) o[p] = __builtin_amdgcn_perm(r[u][2 * p + 1][c >> 1], r[u][2 * p][c >> 1], sel);
          int row = mv * 8 + c;
          st16(lds + row * kRowBytes + ((kg ^ swz(row)) << 4), o);
        }
      } else {
        // 8 k-rows x 4 floats -> 4 rows x 8 floats (two chunks 2kg, 2kg+1).
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 lo = {r[u][0][c], r[u][1][c], r[u][2][c], r[u][3][c]};
          u32x4 hi = {r[u][4][c], r[u][5][c], r[u][6][c], r[u][7][c]};
          int row = mv * 4 + c;
          st16(lds + row * kRowBytes + (((2 * kg) ^ swz(row)) << 4), lo);
          st16(lds + row * kRowBytes + (((2 * kg + 1) ^ swz(row)) << 4), hi);
        }
      }
    }
  }
};

// 8-element k-group `kg` of LDS row `row` as an MFMA fragment.
template <typename T>
__device__ __forceinline__ void lds_frag(Frag8<T>& f, const char* tile, int row, int kg) {
  const char* rp = tile + row * kRowBytes;
  if constexpr (sizeof(T) == 2) {
    load_frag(f, reinterpret_cast<const T*>(rp + ((kg ^ swz(row)) << 4)));
  } else {
    load_frag2(f, reinterpret_cast<const T*>(rp + (((2 * kg) ^ swz(row)) << 4)),
               reinterpret_cast<const T*>(rp + (((2 * kg + 1) ^ swz(row)) << 4)));
  }
}

template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, bool A_K, bool B_K, int EPI, typename TC>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave) void gemm_kernel(Args g) {
  constexpr int NT = WAVES_M * WAVES_N * kWave;
  constexpr int BK = kRowBytes / sizeof(T);
  constexpr int STEPS = BK / 16;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int kStage = (BM + BN) * kRowBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int l32 = lane & 31, grp = lane >> 5;

  // ---- tile order: XCD-contiguous renumbering, then grouped row-major walk
  const int nblk = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
  const int in_group = kGroupM * g.tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsize = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (logical % in_group) % gsize;
  const int tn = (logical % in_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  using LA = typename std::conditional<A_K, KMajorLoader<T, BM, NT>, MNMajorLoader<T, BM, NT>>::type;
  using LB = typename std::conditional<B_K, KMajorLoader<T, BN, NT>, MNMajorLoader<T, BN, NT>>::type;
  LA la;
  LB lb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (g.K + BK - 1) / BK;
  la.load(g.A, g.lda, m0, g.M, 0, g.K, tid);
  lb.load(g.B, g.ldb, n0, g.N, 0, g.K, tid);
  la.store(smem, tid);
  lb.store(smem + BM * kRowBytes, tid);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    char* cur = smem + (kt & 1) * kStage;
    const bool more = kt + 1 < KT;
    if (more) {
      la.load(g.A, g.lda, m0, g.M, (kt + 1) * BK, g.K, tid);
      lb.load(g.B, g.ldb, n0, g.N, (kt + 1) * BK, g.K, tid);
    }
    const char* As = cur;
    const char* Bs = cur + BM * kRowBytes;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      Frag8<T> fa[TM], fb[TN];
      const int kg = 2 * st + grp;
#pragma unroll
      for (int i = 0; i < TM; ++i) lds_frag<T>(fa[i], As, wm * WTM + i * 32 + l32, kg);
#pragma unroll
      for (int j = 0; j < TN; ++j) lds_frag<T>(fb[j], Bs, wn * WTN + j * 32 + l32, kg);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma_step(acc[i][j], fb[j], fa[i]);
    }
    if (more) {
      char* nxt = smem + ((kt + 1) & 1) * kStage;
      la.store(nxt, tid);
      lb.store(nxt + BM * kRowBytes, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: lane owns row m, columns n..n+3 per accumulator quad
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WTM + i * 32 + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * grp;
        if (n >= g.N) continue;
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
          float b[4];
          load4(reinterpret_cast<const T*>(g.bias) + n, b);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += b[e];
        }
        TC* cp = reinterpret_cast<TC*>(g.C) + (int64_t)m * g.ldc + n;
        if constexpr (EPI == EPI_DGELU) {
          float u[4];
          load4(reinterpret_cast<const T*>(g.C2) + (int64_t)m * g.ldc2 + n, u);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= gelu_grad_f(u[e]);
        }
        store4(cp, v[0], v[1], v[2], v[3]);
        if constexpr (EPI == EPI_BIAS_GELU) {
          T* ap = reinterpret_cast<T*>(g.C2) + (int64_t)m * g.ldc2 + n;
          store4(ap, gelu_f(v[0]), gelu_f(v[1]), gelu_f(v[2]), gelu_f(v[3]));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch

struct TileCfg { int bm, bn; };

template <typename T, int BM, int BN, int WM, int WN, bool AK, bool BK_, int EPI, typename TC>
hipError_t run(const GemmDesc& d, hipStream_t s) {
  Args a;
  a.A = static_cast<const char*>(d.A); a.lda = d.lda;
  a.B = static_cast<const char*>(d.B); a.ldb = d.ldb;
  a.C = static_cast<char*>(d.C); a.ldc = d.ldc;
  a.C2 = static_cast<char*>(d.C2); a.ldc2 = d.ldc2;
  a.bias = static_cast<const char*>(d.bias);
  a.M = (int)d.M; a.N = (int)d.N; a.K = (int)d.K;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int nblk = a.tiles_m * a.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, AK, BK_, EPI, TC>), dim3(nblk),
                     dim3(WM * WN * kWave), 0, s, a);
  return hipGetLastError();
}

// Pick the tile that minimises (rounds of workgroups over 256 CUs) x (tile cost).
TileCfg choose_tile(int dtype, int64_t M, int64_t N) {
  if (dtype == DT_F32) return {128, 128};
  struct Cand { int bm, bn, per_cu; double eff; };
  const Cand cands[] = {{256, 256, 1, 1.00}, {256, 128, 1, 0.90}, {128, 128, 2, 0.78}};
  double best = 1e300;
  TileCfg pick{128, 128};
  for (const Cand& c : cands) {
    int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    int64_t rounds = (tiles + 256 * c.per_cu - 1) / (256 * c.per_cu);
    double cost = (double)rounds * c.bm * c.bn / c.eff / c.per_cu;
    if (cost < best * 0.999) { best = cost; pick = {c.bm, c.bn}; }
  }
  return pick;
}

template <typename T, bool AK, bool BK_, int EPI, typename TC>
hipError_t run_tiles(const GemmDesc& d, hipStream_t s) {
  TileCfg t = choose_tile(d.dtype, d.M, d.N);
  if constexpr (sizeof(T) == 4) {
    return run<T, 128, 128, 2, 2, AK, BK_, EPI, TC>(d, s);
  } else {
    if (t.bm == 256 && t.bn == 256) return run<T, 256, 256, 2, 2, AK, BK_, EPI, TC>(d, s);
    if (t.bm == 256 && t.bn == 128) return run<T, 256, 128, 2, 2, AK, BK_, EPI, TC>(d, s);
    return run<T, 128, 128, 2, 2, AK, BK_, EPI, TC>(d, s);
  }
}

template <typename T>
hipError_t dispatch(const GemmDesc& d, hipStream_t s) {
  if (d.a_kmajor && d.b_kmajor) {
    if (d.c_f32) return hipErrorInvalidValue;
    switch (d.epi) {
      case EPI_NONE: return run_tiles<T, true, true, EPI_NONE, T>(d, s);
      case EPI_BIAS: return run_tiles<T, true, true, EPI_BIAS, T>(d, s);
      case EPI_BIAS_GELU: return run_tiles<T, true, true, EPI_BIAS_GELU, T>(d, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (d.a_kmajor && !d.b_kmajor) {
    if (d.c_f32) return hipErrorInvalidValue;
    switch (d.epi) {
      case EPI_NONE: return run_tiles<T, true, false, EPI_NONE, T>(d, s);
      case EPI_DGELU: return run_tiles<T, true, false, EPI_DGELU, T>(d, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (!d.a_kmajor && !d.b_kmajor && d.c_f32 && d.epi == EPI_NONE)
    return run_tiles<T, false, false, EPI_NONE, float>(d, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmDesc& d, hipStream_t s) {
  TraceScope trace(d.a_kmajor && d.b_kmajor ? K_GEMM_NT : (d.a_kmajor ? K_GEMM_NN : K_GEMM_TN), s,
                   2.0 * (double)d.M * (double)d.N * (double)d.K);
  if (d.dtype == DT_BF16) return dispatch<bf16>(d, s);
  return dispatch<float>(d, s);
}

}  // namespace tpl
