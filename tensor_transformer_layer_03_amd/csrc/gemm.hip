// Dense products of the parallel linear layers on gfx950 MFMA.
//
// Every contraction of the layer shard is C[M][N] = sum_k A(m,k) B(n,k):
//   forward  (NT): A = activations [M][K], B = weight [N][K]      (both K-major)
//   dgrad    (NN): A = dY [M][K'],         B = weight [K'][N]     (B N-major)
//   wgrad    (TN): A = dY^T via dY [K][M], B = X via [K][N]       (both MN-major)
// (guide page section 1.2: tensor parallelism splits one matrix product over
// devices; each rank runs its slice through this kernel.)
//
// Kernels (all on v_mfma_f32_32x32x16_bf16 per 16 k; fp32: 8 x
// v_mfma_f32_32x32x2f32). The weight-side fragment is the MFMA's A operand,
// so lane l owns output row m = l%32 and four consecutive columns per
// accumulator quad: epilogue stores are 8/16 B.
//  * gemm_kernel (fp32 storage): 128x128 tile, K-tile of 32 fp32 (128-B LDS
//    rows), MN-major operands loaded as 8 k-rows x 16 B and transposed across
//    lanes before the K-contiguous LDS store;
//  * gemm_bf16_kernel: 256x256 or 256x192 (8 waves) or 128x128 (4 waves) tile, K-tile of
//    64 bf16, two LDS stages; forward operands go straight to LDS
//    (buffer_load ... lds), MN-major operands through registers into an
//    [k][mn] LDS tile read with ds_read_b64_tr_b16; optional deterministic
//    split-K for fp32 weight gradients;
//  * gemm_ms_kernel (forward products only): K-tile of 32 bf16, four LDS
//    stages fed three tiles ahead, with the fused loss-statistics epilogue
//    for the logits.
// Workgroups are renumbered so that consecutive tiles share an XCD (the
// dispatcher deals workgroups to the 8 XCDs round-robin, each with its own
// L2), then walked in groups of kGroupM tile-rows for L2 reuse of B (4 rows
// measured best overall: 2 helps some products and loses 2% on others, 16
// loses 2-3% everywhere).
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <vector>

#include "colsum.h"
#include "common.h"
#include "kernels.h"

namespace tpl {

namespace {

constexpr int kRowBytes = 128;   // one LDS row = one K-tile of one output row/col
constexpr int kGroupM = 4;
constexpr float kLog2e = 1.4426950408889634f;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

struct Args {
  const char* A; int64_t lda;
  const char* B; int64_t ldb;
  char* C; int64_t ldc;
  char* C2; int64_t ldc2;
  const char* bias;
  int M, N, K;
  int tiles_m, tiles_n;
  const int32_t* targets;
  int64_t v0;
  float* xpart;
  float* ws;       // split-K partials [splits-1][M][N] (split 0 writes C)
  int splits, kchunk;
  float* colpart;  // EPI_DGELU: column sums of the output per half tile of rows (or NULL)
  int64_t a_trim;  // bytes of an MN-major A past its last row's M columns that are not the caller's
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
          float gp[4];
          load4(reinterpret_cast<const T*>(g.C2) + (int64_t)m * g.ldc2 + n, gp);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= gp[e];
        }
        if constexpr (EPI == EPI_BIAS_GELU) {
          float ge[4], gp[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) gelu_and_grad(v[e], ge[e], gp[e]);
          store4(cp, gp[0], gp[1], gp[2], gp[3]);
          T* ap = reinterpret_cast<T*>(g.C2) + (int64_t)m * g.ldc2 + n;
          store4(ap, ge[0], ge[1], ge[2], ge[3]);
        } else {
          store4(cp, v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 kernel
// Direct-to-LDS version for bf16: every operand tile goes global -> LDS with
// buffer_load_dwordx4 ... lds (lane l of a wave writes bytes 16l..16l+15 of a
// 1 KB LDS block; the swizzle is produced by choosing which 16 B each lane
// fetches), so no registers or VALU are spent on staging. Reads past the end
// of an operand (num_records of the buffer resource) return zeros.
//  K-major tile  [rows][64 k]: 128 B rows, chunk c of row r at c ^ swz_k(r);
//    a fragment (8 consecutive k of one row) is one ds_read_b128.
//  MN-major tile [64 k][rows]: rows of 2*ROWS bytes, chunk c of row k at
//    c ^ 2*(k & 3); a fragment is two ds_read_b64_tr_b16: within each group of
//    16 lanes the instruction hands lane j element j%4 of the 8 bytes read by
//    lanes j/4, j/4+4, j/4+8, j/4+12, so source lane 4e+q points at row k0+e,
//    columns base+4q..base+4q+3 and lane j receives column base+j, rows
//    k0..k0+3 -- four consecutive k of one output row/column, as the MFMA wants.
//
// Schedule of one K-tile (4 k16-steps, one barrier): the fragments of step
// s+1 are read during the MFMAs of step s; the barrier sits inside step 3,
// and the first fragments of tile kt+1 are read while the rest of step 3's
// MFMAs run. Loads run ahead of the MFMAs so that a tile's global latency
// (HBM when the weights are not cached) is covered by more than one K-tile:
//  * direct-to-LDS: each operand has a ring of 2 or 3 LDS stages; the loads
//    of tile kt+S-1 of an operand with S stages are issued during step 0,
//    and the barrier waits only for tile kt+1 (the deeper tiles stay in
//    flight; loads return in issue order, so the deeper operand is issued
//    last);
//  * register-staged: tile kt+1, loaded into registers during tile kt-1, is
//    written to its LDS stage during step 2 of tile kt, and the loads of tile
//    kt+2 are issued right after, a whole K-tile ahead of their use.
// Past the last tile the loads go to a zero-length buffer.

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((__vector_size__(8)));

// Row swizzle of K-major tiles; depends on r mod 32 only, so the 32-row
// fragments of a wave share one lane pattern.
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 3); }
__device__ __forceinline__ int swz_t(int k) { return 4 * (k & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, n, 0x00020000);
}

// LDS layout of direct-to-LDS K-major tiles ("padded"): 1 KB blocks of 8
// rows x 128 B at a pitch of 1040 B; block b holds rows b%8 + 8p + 64(b/8),
// p = 0..7, at position p, each row's 8 chunks in natural order. A load
// instruction then reads 8 whole 128-B lines in order (one 128-B request per
// line instead of two 64-B ones), and a fragment read of 16 consecutive rows
// at one chunk still lands on 16 distinct 16-B bank groups: row R sits at
// (R%8) * 1040 + ((R/8)%2) * 128 modulo 256.
constexpr int kPadBlk = 1040;
template <int ROWS, bool PAD>
constexpr int tile_bytes() { return PAD ? ROWS / 8 * kPadBlk : ROWS * 128; }
__device__ __forceinline__ int pad_row_off(int r) { return ((r & 7) + 8 * (r >> 6)) * kPadBlk + ((r >> 3) & 7) * 128; }

// Direct-to-LDS loads of one operand tile (ROWS x 64 bf16) for one wave:
// kInst instructions of 1 KB; per-lane byte offsets are fixed over K.
template <int ROWS, bool KMAJ, int NW>
struct TileDma {
  static constexpr bool kKMajor = KMAJ;
  static constexpr int kRows = ROWS;
  static constexpr int kInst = ROWS * 128 / 1024 / NW;
  static_assert(kInst * 1024 * NW == ROWS * 128, "tile does not split evenly over the waves");
  int voff[kInst];
  __device__ __forceinline__ void init(int64_t ld, int row0, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kInst; ++j) {
      const int blk = j * NW + wave;
      if constexpr (KMAJ) {   // padded layout: block blk, position lane/8, chunk lane%8
        const int r = (blk & 7) + 8 * (lane >> 3) + 64 * (blk >> 3);
        voff[j] = (int)(((int64_t)r * ld + (lane & 7) * 8) * 2);
      } else {
        constexpr int kChunks = ROWS / 8, kRowsPerBlk = 64 / kChunks;
        const int k = blk * kRowsPerBlk + lane / kChunks;
        voff[j] = (int)(((int64_t)k * ld + row0 + (((lane % kChunks) ^ swz_t(k)) * 8)) * 2);
      }
    }
  }
  // Loads from a buffer starting at `base` of `bytes` bytes (0: nothing is read,
  // zeros are written). K-major: base = the block's first row, soff = 2*k0.
  // MN-major: base = k-row k0, soff = 0.
  __device__ __forceinline__ void issue(const char* base, int64_t bytes, int soff, char* lds, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)   // the buffer-resource type exists only in the device pass
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < kInst; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (j * NW + wave) * (KMAJ ? kPadBlk : 1024)), 16,
                                               voff[j], soff, 0, 0);
#endif
  }
};

// Register-staged alternative for one operand tile: buffer_load_dwordx4 into
// VGPRs (range-checked, zeros past the operand), then ds_write_b128 into the
// same swizzled LDS layout as the direct-to-LDS path. Used where the compiler
// cannot tell LDS-DMA writes of one stage from transpose reads of the other
// and would otherwise wait for every load before each fragment read.
template <int ROWS, bool KMAJ, int NT>
struct TileReg {
  static constexpr int kPer = ROWS * 8 / NT;   // 16-B chunks per thread
  static_assert(kPer * NT == ROWS * 8, "tile does not split evenly over the threads");
  u32x4 r[kPer];
  int voff[kPer], loff[kPer];
  __device__ __forceinline__ void init(int64_t ld, int row0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = tid + i * NT;
      if constexpr (KMAJ) {
        const int row = p >> 3, c = p & 7;
        voff[i] = (int)(((int64_t)row * ld + c * 8) * 2);
        loff[i] = row * 128 + ((c ^ swz_k(row)) << 4);
      } else {
        constexpr int kC = ROWS / 8;
        const int k = p / kC, c = p % kC;
        voff[i] = (int)(((int64_t)k * ld + row0 + c * 8) * 2);
        loff[i] = k * (ROWS * 2) + ((c ^ swz_t(k)) << 4);
      }
    }
  }
  __device__ __forceinline__ void load(const char* base, int64_t bytes, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)   // the buffer-resource type exists only in the device pass
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < kPer; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], soff, 0);
#endif
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) st16(lds + loff[i], r[i]);
  }
};

// Buffer arguments (base, bytes, scalar offset) of K-tile KT_ of A and of B;
// past the last tile the buffers are zero-length (nothing is read, zeros are
// produced).
// K-major operands: the range ends at the last valid element of the tile's
// last row (((rows - 1) * ld + K) elements from the first row's start), so
// the reads of a ragged last K-tile stop at the operand's end also when a
// K split has moved the base K columns in.
#define TPL_TILE_ARGS_A(KT_)                                                                              \
  (A_K ? g.A + (int64_t)m0 * g.lda * 2 : g.A + (int64_t)(KT_) * 64 * g.lda * 2),                         \
      ((KT_) * 64 < g.K ? (A_K ? ((int64_t)(g.M - m0 - 1) * g.lda + g.K) * 2                            \
                               : (int64_t)(g.K - (KT_) * 64) * g.lda * 2 - g.a_trim)                      \
                        : 0),                                                                            \
      (A_K ? (KT_) * 128 : 0)
#define TPL_TILE_ARGS_B(KT_)                                                                              \
  (B_K ? g.B + (int64_t)n0 * g.ldb * 2 : g.B + (int64_t)(KT_) * 64 * g.ldb * 2),                         \
      ((KT_) * 64 < g.K ? (B_K ? ((int64_t)(g.N - n0 - 1) * g.ldb + g.K) * 2                            \
                               : (int64_t)(g.K - (KT_) * 64) * g.ldb * 2)                                 \
                        : 0),                                                                            \
      (B_K ? (KT_) * 128 : 0)

// Fragment of tile row r0 + lane%32, k-slots 8*(lane/32)..+7 of step st.
template <int ROWS, bool KMAJ, bool PAD>
__device__ __forceinline__ void frag_v2(Frag8<bf16>& f, const char* tile, int r0, int st, int lane) {
  if constexpr (KMAJ && PAD) {
    const int r = r0 + (lane & 31);
    load_frag(f, reinterpret_cast<const bf16*>(tile + pad_row_off(r) + (2 * st + (lane >> 5)) * 16));
  } else if constexpr (KMAJ) {
    const int r = r0 + (lane & 31);
    const int c = (2 * st + (lane >> 5)) ^ swz_k(r);
    load_frag(f, reinterpret_cast<const bf16*>(tile + r * 128 + c * 16));
  } else {
    const int G = lane >> 4, s = lane & 15, e = s >> 2, q = s & 3;
    const int mn = r0 + 16 * (G & 1) + 4 * q;
    const int k = 16 * st + 8 * (G >> 1) + e;
    const int c0 = (mn >> 3) ^ swz_t(k);   // swz_t(k) == swz_t(k + 4)
    const char* p0 = tile + k * (ROWS * 2) + c0 * 16 + (q & 1) * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0 + 4 * ROWS * 2));
    __builtin_memcpy(reinterpret_cast<char*>(&f.v), &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&f.v) + 8, &hi, 8);
  }
}

// Fragments of step st for a wave's TM row tiles (A) and TN column tiles (B),
// from an A and a B stage.
template <int BM, int BN, bool A_K, bool B_K, bool PAD, int TM, int TN>
__device__ __forceinline__ void read_frags2(Frag8<bf16> (&fa)[TM], Frag8<bf16> (&fb)[TN], const char* sa,
                                            const char* sb, int st, int arow, int brow, int lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i) frag_v2<BM, A_K, PAD>(fa[i], sa, arow + i * 32, st, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) frag_v2<BN, B_K, PAD>(fb[j], sb, brow + j * 32, st, lane);
}

template <int TM, int TN>
__device__ __forceinline__ void mfma_tile(f32x16 (&acc)[TM][TN], const Frag8<bf16> (&fa)[TM],
                                          const Frag8<bf16> (&fb)[TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) mfma_step(acc[i][j], fb[j], fa[i]);
}

__device__ __forceinline__ void zero_frag(Frag8<bf16>& f) {
  u32x4 z = {0u, 0u, 0u, 0u};
  __builtin_memcpy(&f.v, &z, 16);
}

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt low bits 3:0, high
// bits 15:14; expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// Bias of a lane's output columns (TN blocks of 32 x 4 quads x 4 values,
// the accumulator layout), loaded once per tile as packed bf16 pairs through
// a buffer resource: columns at or past N read 0, so there is no branch and
// every load is in flight at once.
template <int TN>
struct BiasCols {
  u32x2 pk[TN][4];
  __device__ __forceinline__ void load(const char* bias, int N, int ncol0, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)   // the buffer-resource type exists only in the device pass
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(bias, (int64_t)N * 2);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pk[j][q] = __builtin_amdgcn_raw_buffer_load_b64(rs, (ncol0 + j * 32 + 8 * q + 4 * (lane >> 5)) * 2, 0, 0);
#endif
  }
  __device__ __forceinline__ void add(float* v, int j, int q) const {
    v[0] += __builtin_bit_cast(float, pk[j][q][0] << 16);
    v[1] += __builtin_bit_cast(float, pk[j][q][0] & 0xFFFF0000u);
    v[2] += __builtin_bit_cast(float, pk[j][q][1] << 16);
    v[3] += __builtin_bit_cast(float, pk[j][q][1] & 0xFFFF0000u);
  }
};

// Output tile staged through LDS: the waves write their values (4
// consecutive columns per lane and accumulator quad) into an LDS copy of the
// tile's rows, 16-B chunks XOR-swizzled by row; then every thread copies whole
// 16-B chunks of whole rows to global memory, so a wave's store covers full
// 128-B lines (a direct store from the MFMA layout touches 32 rows with 16 B
// each, and the memory pipeline pays per line).
template <typename TC, int BN, int NT>
struct CStage {
  static constexpr int kRowBytes = BN * (int)sizeof(TC);
  static constexpr int kChunks = kRowBytes / 16;
  // XOR range: the largest power of two dividing the row's chunk count (at
  // most 32), so a swizzled chunk stays inside its row
  static constexpr int kSwz = ((kChunks & -kChunks) < 32 ? (kChunks & -kChunks) : 32) - 1;
  __device__ __forceinline__ static int off(int r, int c) {   // column c (a multiple of 4) of staged row r
    const int byte = c * (int)sizeof(TC);
    return r * kRowBytes + (((byte >> 4) ^ (r & kSwz)) << 4) + (byte & 15);
  }
  __device__ __forceinline__ static void put4(char* lds, int r, int c, const float* v) {
    if constexpr (sizeof(TC) == 2) {
      store4(reinterpret_cast<bf16*>(lds + off(r, c)), v[0], v[1], v[2], v[3]);
    } else {
      *reinterpret_cast<f32x4*>(lds + off(r, c)) = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
  __device__ __forceinline__ static void get4(const char* lds, int r, int c, float* v) {
    static_assert(sizeof(TC) == 2, "bf16 tiles only");
    load4(reinterpret_cast<const bf16*>(lds + off(r, c)), v);
  }
  // C2 rows m0.., columns n0.. -> staged rows [0, ROWS) (whole 16-B chunks of
  // whole rows, all loads in flight before the LDS writes); out of range
  // reads as 0
  template <int ROWS>
  __device__ __forceinline__ static void fill(char* lds, const char* src, int64_t ld, int m0, int n0, int M, int N,
                                              int tid) {
    constexpr int kPer = ROWS * kChunks / NT;
    static_assert(kPer * NT == ROWS * kChunks, "staged rows do not split evenly over the threads");
    constexpr int kBatch = kPer < 4 ? kPer : 4;
#pragma unroll
    for (int b0 = 0; b0 < kPer; b0 += kBatch) {
      u32x4 v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int idx = tid + (b0 + b) * NT;
        const int r = idx / kChunks, ch = idx % kChunks;
        const int m = m0 + r, n = n0 + ch * (16 / (int)sizeof(TC));
        v[b] = u32x4{0u, 0u, 0u, 0u};
        if (m < M && n < N) v[b] = *reinterpret_cast<const u32x4*>(src + ((int64_t)m * ld + n) * (int)sizeof(TC));
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int idx = tid + (b0 + b) * NT;
        const int r = idx / kChunks, ch = idx % kChunks;
        *reinterpret_cast<u32x4*>(lds + r * kRowBytes + ((ch ^ (r & kSwz)) << 4)) = v[b];
      }
    }
  }
  // staged rows [0, rows) -> C rows m0.., columns n0..
  __device__ __forceinline__ static void flush(const char* lds, int rows, char* C, int64_t ldc, int m0, int n0, int M,
                                               int N, int tid) {
    for (int idx = tid; idx < rows * kChunks; idx += NT) {
      const int r = idx / kChunks, ch = idx % kChunks;
      const int m = m0 + r, n = n0 + ch * (16 / (int)sizeof(TC));
      if (m < M && n < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * kRowBytes + ((ch ^ (r & kSwz)) << 4));
        *reinterpret_cast<u32x4*>(C + ((int64_t)m * ldc + n) * (int)sizeof(TC)) = v;
      }
    }
  }
};

// LDS stages of the A and B tiles. Direct-to-LDS forward tiles keep a third
// stage of the weight operand (B) where the LDS holds it: its rows come from
// HBM when the weights are not cached, the activations (A) usually from the
// caches. 256x192: 2 + 3 stages, 141 KB (measured on the 175B rank's forward
// products: 10% faster from cold caches, level from warm ones); 256x128: 3 +
// 3 stages, 146 KB. The 256x256 and 128x128 tiles keep 2 + 2 (a third stage
// does not fit, or would halve the workgroups per CU).
template <int BM, int BN, bool DMA>
constexpr int stages_a() { return DMA && BM == 256 && BN == 128 ? 3 : 2; }
template <int BM, int BN, bool DMA>
constexpr int stages_b() { return DMA && BM == 256 && (BN == 192 || BN == 128) ? 3 : 2; }
// LDS of one workgroup of the two-stage kernel: the A stages, then the B stages.
template <int BM, int BN, bool DMA>
constexpr int body_smem_bytes() {
  return stages_a<BM, BN, DMA>() * tile_bytes<BM, DMA>() + stages_b<BM, BN, DMA>() * tile_bytes<BN, DMA>();
}

// s_waitcnt with a vmcnt limit and lgkmcnt(0) (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// One output tile (workgroup number bid of the product's grid); smem holds
// body_smem_bytes<BM, BN, DMA>() bytes.
template <int BM, int BN, int WGM, int WGN, bool A_K, bool B_K, bool DMA, int EPI, typename TC>
__device__ __forceinline__ void gemm_bf16_body(Args g, int bid, char* smem) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, TM = WTM / 32, TN = WTN / 32;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WGM, wn = wave / WGM;

  const int nblk = g.tiles_m * g.tiles_n;
  if (g.splits > 1) {
    // split-K: workgroup (split, tile) takes K range [split*kchunk, ...);
    // split 0 writes C, split s the workspace slice s-1 (summed afterwards
    // in split order)
    const int split = bid / nblk;
    bid -= split * nblk;
    const int kb = split * g.kchunk;
    g.A += A_K ? (int64_t)kb * 2 : (int64_t)kb * g.lda * 2;
    g.B += B_K ? (int64_t)kb * 2 : (int64_t)kb * g.ldb * 2;
    g.K = min(g.kchunk, g.K - kb);
    if (split > 0) {
      g.C = reinterpret_cast<char*>(g.ws + (int64_t)(split - 1) * g.M * g.N);
      g.ldc = g.N;
    }
  }
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
  const int in_group = kGroupM * g.tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsize = min(g.tiles_m - first_m, kGroupM);
  const int m0 = (first_m + (logical % in_group) % gsize) * BM;
  const int n0 = ((logical % in_group) / gsize) * BN;

  using LA = typename std::conditional<DMA, TileDma<BM, A_K, WGM * WGN>, TileReg<BM, A_K, WGM * WGN * 64>>::type;
  using LB = typename std::conditional<DMA, TileDma<BN, B_K, WGM * WGN>, TileReg<BN, B_K, WGM * WGN * 64>>::type;
  LA tA;
  LB tB;
  if constexpr (DMA) {
    tA.init(g.lda, A_K ? 0 : m0, wave, lane);
    tB.init(g.ldb, B_K ? 0 : n0, wave, lane);
  } else {
    tA.init(g.lda, A_K ? 0 : m0, (int)threadIdx.x);
    tB.init(g.ldb, B_K ? 0 : n0, (int)threadIdx.x);
  }


  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Frag8<bf16> fa[2][TM], fb[2][TN];
  constexpr int kMf = TM * TN;                                // MFMAs per step
  constexpr int kRd = (TM + TN) * (A_K && B_K ? 1 : 2);        // LDS read instructions per step (upper bound)
  constexpr int kVm = DMA ? TileDma<BM, A_K, WGM * WGN>::kInst + TileDma<BN, B_K, WGM * WGN>::kInst
                          : TileReg<BM, A_K, WGM * WGN * 64>::kPer + TileReg<BN, B_K, WGM * WGN * 64>::kPer;

  const int KT = g.K / 64;                  // full K-tiles; a partial last tile is handled after the loop
  const int ktail = g.K & 63;
  constexpr int SA = stages_a<BM, BN, DMA>(), SB = stages_b<BM, BN, DMA>();
  static_assert(SA >= 2 && SB >= 2 && SA - SB <= 1 && SB - SA <= 1 && (DMA || (SA == 2 && SB == 2)),
                "stage rings differ by at most one stage; register staging keeps two");
  constexpr int kTA = tile_bytes<BM, DMA>(), kTB = tile_bytes<BN, DMA>();
  // DMA loads of the deeper tiles that may stay in flight at a barrier
  constexpr int kWait = DMA ? TileDma<BM, A_K, NW>::kInst * (SA - 2) + TileDma<BN, B_K, NW>::kInst * (SB - 2) : 0;
  const auto stA = [&](int t) { return smem + (t % SA) * kTA; };
  const auto stB = [&](int t) { return smem + SA * kTA + (t % SB) * kTB; };
#define TPL_LOAD_A(T_) tA.load(TPL_TILE_ARGS_A(T_))
#define TPL_LOAD_B(T_) tB.load(TPL_TILE_ARGS_B(T_))
#define TPL_DMA_A(T_) tA.issue(TPL_TILE_ARGS_A(T_), stA(T_), wave)
#define TPL_DMA_B(T_) tB.issue(TPL_TILE_ARGS_B(T_), stB(T_), wave)

  if constexpr (DMA) {
#pragma unroll
    for (int t = 0; t < (SA > SB ? SA : SB) - 1; ++t) {
      if (SA > SB) {   // the deeper ring's loads last
        if (t <= SB - 2) TPL_DMA_B(t);
        if (t <= SA - 2) TPL_DMA_A(t);
      } else {
        if (t <= SA - 2) TPL_DMA_A(t);
        if (t <= SB - 2) TPL_DMA_B(t);
      }
    }
    wait_vm_lgkm<kWait>();   // tile 0 has landed
  } else {
    TPL_LOAD_A(0);
    TPL_LOAD_B(0);
    tA.store(stA(0));
    tB.store(stB(0));
    TPL_LOAD_A(1);
    TPL_LOAD_B(1);
    wait_vm_lgkm<63>();      // this wave's LDS writes are done (tile 1 stays in flight)
  }
  __builtin_amdgcn_s_barrier();
  read_frags2<BM, BN, A_K, B_K, DMA, TM, TN>(fa[0], fb[0], stA(0), stB(0), 0, wm * WTM, wn * WTN, lane);

  for (int kt = 0; kt < KT; ++kt) {
    // direct-to-LDS tiles: the wave's compute phase at raised issue priority,
    // its wait for the next tile at the default (forward products 2-4%
    // faster; level on the register-staged paths, which keep the default)
    if constexpr (DMA) __builtin_amdgcn_s_setprio(1);
    const char* ca = stA(kt);
    const char* cb = stB(kt);
    // step 0: fragments of step 1 (first, so no LDS write is ordered before
    // them), then (direct-to-LDS) the loads of the tiles ahead, around this
    // step's MFMAs
    read_frags2<BM, BN, A_K, B_K, DMA, TM, TN>(fa[1], fb[1], ca, cb, 1, wm * WTM, wn * WTN, lane);
    if constexpr (DMA) {
      if (SA > SB) {
        TPL_DMA_B(kt + SB - 1);
        TPL_DMA_A(kt + SA - 1);
      } else {
        TPL_DMA_A(kt + SA - 1);
        TPL_DMA_B(kt + SB - 1);
      }
    }
    mfma_tile<TM, TN>(acc, fa[0], fb[0]);
#pragma unroll
    for (int x = 0; x < kMf; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (x < kRd) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      if (DMA && x < kVm) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
    }
    // steps 1, 2
    read_frags2<BM, BN, A_K, B_K, DMA, TM, TN>(fa[0], fb[0], ca, cb, 2, wm * WTM, wn * WTN, lane);
    mfma_tile<TM, TN>(acc, fa[1], fb[1]);
#pragma unroll
    for (int x = 0; x < kMf; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (x < kRd) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    read_frags2<BM, BN, A_K, B_K, DMA, TM, TN>(fa[1], fb[1], ca, cb, 3, wm * WTM, wn * WTN, lane);
    if constexpr (!DMA) {   // stage kt+1 is free since the last barrier; then tile kt+2 into the registers
      tA.store(stA(kt + 1));
      tB.store(stB(kt + 1));
      TPL_LOAD_A(kt + 2);
      TPL_LOAD_B(kt + 2);
    }
    mfma_tile<TM, TN>(acc, fa[0], fb[0]);
#pragma unroll
    for (int x = 0; x < kMf; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (x < kRd) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      if (!DMA && x < kVm) __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 1, 0);
      if (!DMA && x < kVm) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
    }
    // step 3: a few MFMAs, then sync on the next tile, then its first fragments
    // are read while the remaining MFMAs of this step run
    constexpr int kHead = kMf / 4;
#pragma unroll
    for (int x = 0; x < kHead; ++x) mfma_step(acc[x / TN][x % TN], fb[1][x % TN], fa[1][x / TN]);
    // tile kt+1 has landed in this wave's share (direct-to-LDS) or been written
    // (registers), and its fragment reads are done; then every other wave's
    if constexpr (DMA) __builtin_amdgcn_s_setprio(0);
    wait_vm_lgkm<DMA ? kWait : 63>();
    __builtin_amdgcn_s_barrier();
    read_frags2<BM, BN, A_K, B_K, DMA, TM, TN>(fa[0], fb[0], stA(kt + 1), stB(kt + 1), 0, wm * WTM, wn * WTN, lane);
#pragma unroll
    for (int x = kHead; x < kMf; ++x) mfma_step(acc[x / TN][x % TN], fb[1][x % TN], fa[1][x / TN]);
#pragma unroll
    for (int x = kHead; x < kMf; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (x - kHead < kRd) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
  }
  if (ktail) {
    // partial last tile (in its stage since the last loop barrier, or the
    // prologue's when K < 64): k-slots at or past K contribute zero
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st > 0)
        read_frags2<BM, BN, A_K, B_K, DMA, TM, TN>(fa[0], fb[0], stA(KT), stB(KT), st, wm * WTM, wn * WTN, lane);
      if (KT * 64 + 16 * st + 8 * (lane >> 5) >= g.K) {
#pragma unroll
        for (int i = 0; i < TM; ++i) zero_frag(fa[0][i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) zero_frag(fb[0][j]);
      }
      mfma_tile<TM, TN>(acc, fa[0], fb[0]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load past the last tile is still in flight
#undef TPL_LOAD_A
#undef TPL_LOAD_B
#undef TPL_DMA_A
#undef TPL_DMA_B

  // epilogue through LDS (the stages are free once every wave is past its
  // last fragment read); fp32 tiles that exceed the LDS go in row passes
  using Stage = CStage<TC, BN, NW * 64>;
  constexpr int kCap = body_smem_bytes<BM, BN, DMA>() / Stage::kRowBytes;   // rows the LDS holds
  constexpr int kRP = kCap >= BM ? BM : (kCap >= 128 ? 128 : (kCap >= 64 ? 64 : 32));
  static_assert(kRP >= WTM && BM % kRP == 0 && kRP % WTM == 0, "staging rows must hold whole wave tiles");
  // GeLU epilogue: round 0 stages GeLU'(u) and leaves GeLU(u) in the
  // accumulators, round 1 stages those
  constexpr int kRounds = EPI == EPI_BIAS_GELU ? 2 : 1;
  BiasCols<TN> bias;
  if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) bias.load(g.bias, g.N, n0 + wn * WTN, lane);
  __syncthreads();
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
#pragma unroll
    for (int p = 0; p < BM / kRP; ++p) {
      if constexpr (EPI == EPI_DGELU) {   // the pass's rows of u, staged where the results go
        Stage::template fill<kRP>(smem, g.C2, g.ldc2, m0 + p * kRP, n0, g.M, g.N, (int)threadIdx.x);
        __syncthreads();
      }
      if ((wm * WTM) / kRP == p) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int rt = wm * WTM + i * 32 + (lane & 31);   // row within the tile
#pragma unroll
          for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nt = wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
              float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              if constexpr (EPI == EPI_BIAS) bias.add(v, j, q);
              if constexpr (EPI == EPI_DGELU) {
                float gp[4];
                Stage::get4(smem, rt - p * kRP, nt, gp);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= gp[e];
              }
              if constexpr (EPI == EPI_BIAS_GELU) {
                if (round == 0) {
                  bias.add(v, j, q);
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    float ge, gp;
                    gelu_and_grad(v[e], ge, gp);
                    acc[i][j][4 * q + e] = ge;
                    v[e] = gp;
                  }
                }
              }
              Stage::put4(smem, rt - p * kRP, nt, v);
            }
          }
        }
      }
      __syncthreads();
      if constexpr (EPI == EPI_DGELU && sizeof(TC) == 2) {
        // column sums of the staged (rounded) rows: thread t takes column
        // t % BN over row block t / BN (kRC rows) of the tile, rows in order
        constexpr int kH = NW * 64 / BN, kRC = BM / kH;
        static_assert(kRP == BM && kH * BN == NW * 64 && kH * kRC == BM, "one staged pass, whole row blocks");
        if (g.colpart) {
          const int c = (int)threadIdx.x % BN, h = (int)threadIdx.x / BN;
          const int rend = min(kRC, g.M - m0 - h * kRC);
          if (rend > 0) {
            float sum = 0.f;
            for (int r = 0; r < rend; ++r)
              sum += (float)*reinterpret_cast<const bf16*>(smem + Stage::off(h * kRC + r, c));
            if (n0 + c < g.N) g.colpart[(int64_t)(m0 / kRC + h) * g.N + n0 + c] = sum;
          }
        }
      }
      Stage::flush(smem, kRP, round == 0 ? g.C : g.C2, round == 0 ? g.ldc : g.ldc2, m0 + p * kRP, n0, g.M, g.N,
                   (int)threadIdx.x);
      __syncthreads();
    }
  }
}

template <int BM, int BN, int WGM, int WGN, bool A_K, bool B_K, bool DMA, int EPI, typename TC>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_bf16_kernel(Args g) {
  __shared__ __attribute__((aligned(1024))) char smem[body_smem_bytes<BM, BN, DMA>()];
  gemm_bf16_body<BM, BN, WGM, WGN, A_K, B_K, DMA, EPI, TC>(g, blockIdx.x, smem);
}

// Two independent products of a block's backward in one launch, both on the
// 256x256 eight-wave tile with register-staged operands: workgroups [0, n0)
// take product 0's tiles (the longer ones in K, so they start first),
// [n0pad, n0pad + tiles of product 1) product 1's. n0pad is n0 rounded up to
// a multiple of 8 (the padding workgroups exit at once) so that both products
// keep their XCD-aware tile walk. One grid lets the short tiles of one product
// fill the compute units the other leaves idle in its last round.
template <int WGM0, int WGN0, bool AK0, bool BK0, int EPI0, typename TC0, int WGM1, int WGN1, bool AK1, bool BK1,
          int EPI1, typename TC1>
__global__ __launch_bounds__(512) void gemm_pair_kernel(Args g0, Args g1, int n0, int n0pad) {
  static_assert(WGM0 * WGN0 == 8 && WGM1 * WGN1 == 8, "both products take 8 waves");
  __shared__ __attribute__((aligned(1024))) char smem[body_smem_bytes<256, 256, false>()];
  const int bid = blockIdx.x;
  if (bid < n0pad) {
    if (bid >= n0) return;
    gemm_bf16_body<256, 256, WGM0, WGN0, AK0, BK0, false, EPI0, TC0>(g0, bid, smem);
  } else {
    gemm_bf16_body<256, 256, WGM1, WGN1, AK1, BK1, false, EPI1, TC1>(g1, bid - n0pad, smem);
  }
}

// The same pairing on 128x128 tiles (four waves, 64 KB of LDS: two
// workgroups per CU), for products whose widths are not multiples of 256 or
// whose 256x256 grid is too coarse to balance; activation gradients without
// an epilogue only.
template <bool AK0, bool BK0, typename TC0, bool AK1, bool BK1, typename TC1>
__global__ __launch_bounds__(256) void gemm_pair128_kernel(Args g0, Args g1, int n0, int n0pad) {
  __shared__ __attribute__((aligned(1024))) char smem[body_smem_bytes<128, 128, false>()];
  const int bid = blockIdx.x;
  if (bid < n0pad) {
    if (bid >= n0) return;
    gemm_bf16_body<128, 128, 2, 2, AK0, BK0, false, EPI_NONE, TC0>(g0, bid, smem);
  } else {
    gemm_bf16_body<128, 128, 2, 2, AK1, BK1, false, EPI_NONE, TC1>(g1, bid - n0pad, smem);
  }
}

// The same product as the first pass of a tail split (the last tile rows
// split over K into fp32 partials); a symbol of its own so that a kernel
// trace tells the two passes apart.
template <int BM, int BN, int WGM, int WGN, bool A_K, bool B_K, bool DMA, int EPI, typename TC>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_bf16_tail_kernel(Args g) {
  __shared__ __attribute__((aligned(1024))) char smem[body_smem_bytes<BM, BN, DMA>()];
  gemm_bf16_body<BM, BN, WGM, WGN, A_K, B_K, DMA, EPI, TC>(g, blockIdx.x, smem);
}

// ------------------------------------------- multi-stage K pipeline (K-major operands)
// Forward (both operands K-major) products with a deeper prefetch: K-tiles of
// 32 (64-B LDS rows), NS LDS stages, loads issued NS-1 tiles ahead straight
// into LDS, and a partial wait (the NS-2 younger tiles stay in flight) before
// the one barrier per K-tile. Four waves in a 2x2 grid. Row r of a 64-B-row
// tile keeps chunk c at c ^ ((r >> 2) & 3): 16 consecutive rows, one chunk ->
// 16 distinct 16-B bank groups.
template <int ROWS, int NW>
struct DmaK32 {   // ROWS x 64 B over NW waves: ROWS/(16 NW) instructions of 1 KB per wave
  static constexpr int kInst = ROWS / (16 * NW);
  int voff[kInst];
  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kInst; ++j) {
      const int r = 16 * (NW * j + wave) + (lane >> 2);
      voff[j] = (int)(((int64_t)r * ld + (((lane & 3) ^ ((r >> 2) & 3)) << 3)) * 2);
    }
  }
  __device__ __forceinline__ void issue(const char* base, int64_t bytes, int soff, char* lds, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)   // the buffer-resource type exists only in the device pass
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < kInst; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (NW * j + wave) * 1024), 16, voff[j], soff, 0, 0);
#endif
  }
};

template <int TM, int TN>
__device__ __forceinline__ void ms_read(Frag8<bf16> (&fa)[TM], Frag8<bf16> (&fb)[TN], const char* a, const char* b) {
#pragma unroll
  for (int i = 0; i < TM; ++i) load_frag(fa[i], reinterpret_cast<const bf16*>(a + i * 2048));
#pragma unroll
  for (int j = 0; j < TN; ++j) load_frag(fb[j], reinterpret_cast<const bf16*>(b + j * 2048));
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 32) asm volatile("s_waitcnt vmcnt(32) lgkmcnt(0)" ::: "memory");
  else static_assert(N < 0, "unsupported wait count");
}

// Fused cross-entropy statistics of a wave's TM x TN fragment block (rows
// rb + 32i + lane%32, columns nb + ...): rounds to bf16 once, stores the
// packed values, and writes per row (max, sum exp(l - max)) over the wave's
// columns to xs[row within the tile]. FULL: every column is below N.
template <int TM, int TN, bool FULL, int BM, int BN>
__device__ __forceinline__ void xent_tile_stats(const Args& g, f32x16 (&acc)[TM][TN], float (&xs)[BM][2], char* stg,
                                                int n0, int nb, int rb, int lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int rt = rb + i * 32 + (lane & 31);
    uint32_t pk[TN][8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const f32x2 pair = {acc[i][j][2 * h], acc[i][j][2 * h + 1]};
        pk[j][h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));   // one v_cvt_pk_bf16_f32
        const float x0 = __builtin_bit_cast(float, pk[j][h] << 16);
        const float x1 = __builtin_bit_cast(float, pk[j][h] & 0xFFFF0000u);
        if constexpr (FULL) {
          mx = fmaxf(mx, fmaxf(x0, x1));
        } else {
          const int n = nb + j * 32 + 8 * (h >> 1) + 4 * (lane >> 5) + 2 * (h & 1);
          if (n < g.N) mx = fmaxf(mx, x0);
          if (n + 1 < g.N) mx = fmaxf(mx, x1);
        }
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float se = 0.f;
    if (mx != -INFINITY) {
      const float off = mx * kLog2e;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          // v_exp_f32 directly: arguments are <= 0 and results below the
          // normal range are negligible in the sum
          const float e0 = __builtin_amdgcn_exp2f(fmaf(__builtin_bit_cast(float, pk[j][h] << 16), kLog2e, -off));
          const float e1 =
              __builtin_amdgcn_exp2f(fmaf(__builtin_bit_cast(float, pk[j][h] & 0xFFFF0000u), kLog2e, -off));
          if constexpr (FULL) {
            se += e0 + e1;
          } else {
            const int n = nb + j * 32 + 8 * (h >> 1) + 4 * (lane >> 5) + 2 * (h & 1);
            if (n < g.N) se += e0;
            if (n + 1 < g.N) se += e1;
          }
        }
    }
    se += __shfl_xor(se, 32, kWave);
    if (lane < 32) {
      xs[rt][0] = mx;
      xs[rt][1] = se;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nt = nb - n0 + j * 32 + 8 * q + 4 * (lane >> 5);   // column within the tile
        u32x2 v = {pk[j][2 * q], pk[j][2 * q + 1]};
        *reinterpret_cast<u32x2*>(stg + CStage<bf16, BN, 64>::off(rt, nt)) = v;
      }
  }
}


template <int BM, int BN, int WGM, int WGN, int NS, int OCC, int EPI, typename TC>
__global__ __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void gemm_ms_kernel(Args g) {
  constexpr int NW = WGM * WGN;
  constexpr int kStage = (BM + BN) * 64, kB = BM * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 fragments per wave
  constexpr int kMf = TM * TN, kRd = TM + TN;
  constexpr int kVm = DmaK32<BM, NW>::kInst + DmaK32<BN, NW>::kInst;   // loads per K-tile per wave
  static_assert((NS & (NS - 1)) == 0 && NS >= 2, "stage count must be a power of two");
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;

  const int nblk = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
  const int in_group = kGroupM * g.tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsize = min(g.tiles_m - first_m, kGroupM);
  const int m0 = (first_m + (logical % in_group) % gsize) * BM;
  const int n0 = ((logical % in_group) / gsize) * BN;

  DmaK32<BM, NW> tA;
  DmaK32<BN, NW> tB;
  tA.init(g.lda, wave, lane);
  tB.init(g.ldb, wave, lane);
  const char* baseA = g.A + (int64_t)m0 * g.lda * 2;
  const char* baseB = g.B + (int64_t)n0 * g.ldb * 2;
  // ranges end at the last valid element of the tile's last row (a ragged last
  // K-tile reads nothing past the operand)
  const int64_t bytesA = ((int64_t)(g.M - m0 - 1) * g.lda + g.K) * 2;
  const int64_t bytesB = ((int64_t)(g.N - n0 - 1) * g.ldb + g.K) * 2;
#define TPL_MS_ISSUE(KT_)                                                                                \
  do {                                                                                                   \
    const bool live_ = (KT_) * 32 < g.K;                                                                 \
    char* s_ = smem + ((KT_) & (NS - 1)) * kStage;                                                       \
    tA.issue(baseA, live_ ? bytesA : 0, (KT_) * 64, s_, wave);                                           \
    tB.issue(baseB, live_ ? bytesB : 0, (KT_) * 64, s_ + kB, wave);                                      \
  } while (0)

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int rl = lane & 31;
  const int aoff = (wm * WTM + rl) * 64, boff = kB + (wn * WTN + rl) * 64;
  const int cx0 = ((lane >> 5) ^ ((rl >> 2) & 3)) << 4, cx1 = ((2 + (lane >> 5)) ^ ((rl >> 2) & 3)) << 4;
  Frag8<bf16> fa[2][TM], fb[2][TN];

  const int KT = g.K / 32;   // full K-tiles; a partial last tile is handled after the loop
  const int ktail = g.K & 31;

#pragma unroll
  for (int t = 0; t < NS - 1; ++t) TPL_MS_ISSUE(t);
  wait_vm_lgkm0<(NS - 2) * kVm>();   // tile 0 has landed (the younger ones may be in flight)
  __builtin_amdgcn_s_barrier();
  ms_read<TM, TN>(fa[0], fb[0], smem + aoff + cx0, smem + boff + cx0);
  __builtin_amdgcn_sched_barrier(0);

  for (int kt = 0; kt < KT; ++kt) {
    const char* cur = smem + (kt & (NS - 1)) * kStage;
    const char* nxt = smem + ((kt + 1) & (NS - 1)) * kStage;
    // step 0: second k-step's fragments and the loads of tile kt+NS-1 around
    // the first k-step's MFMAs (that stage was last read before the previous
    // barrier)
    ms_read<TM, TN>(fa[1], fb[1], cur + aoff + cx1, cur + boff + cx1);
    TPL_MS_ISSUE(kt + NS - 1);
    mfma_tile<TM, TN>(acc, fa[0], fb[0]);
#pragma unroll
    for (int x = 0; x < kMf; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (x < kRd) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      if (x < kVm) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 1: a few MFMAs, then wait for tile kt+1 (the younger tiles stay in
    // flight) and for this wave's reads of `cur`, barrier, then the next
    // tile's first fragments under the remaining MFMAs
    constexpr int kHead = kMf / 8 > 0 ? kMf / 8 : 1;
#pragma unroll
    for (int x = 0; x < kHead; ++x) mfma_step(acc[x / TN][x % TN], fb[1][x % TN], fa[1][x / TN]);
    wait_vm_lgkm0<(NS - 2) * kVm>();
    __builtin_amdgcn_s_barrier();
    ms_read<TM, TN>(fa[0], fb[0], nxt + aoff + cx0, nxt + boff + cx0);
#pragma unroll
    for (int x = kHead; x < kMf; ++x) mfma_step(acc[x / TN][x % TN], fb[1][x % TN], fa[1][x / TN]);
#pragma unroll
    for (int x = kHead; x < kMf; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (x - kHead < kRd) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (ktail) {
    // partial last tile (landed and barriered by the last iteration or the
    // prologue): k-slots at or past K contribute zero
    const char* cur = smem + (KT & (NS - 1)) * kStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks > 0) ms_read<TM, TN>(fa[0], fb[0], cur + aoff + cx1, cur + boff + cx1);
      if (KT * 32 + 16 * ks + 8 * (lane >> 5) >= g.K) {
#pragma unroll
        for (int i = 0; i < TM; ++i) zero_frag(fa[0][i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) zero_frag(fb[0][j]);
      }
      mfma_tile<TM, TN>(acc, fa[0], fb[0]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS at exit
#undef TPL_MS_ISSUE

  if constexpr (EPI == EPI_XENT) {
    // Logits tile (rounded once to bf16 and stored from the packed pairs)
    // plus, per row, the statistics of its BN columns over the stored values:
    // max and sum of exp(l - max). Lanes l and l^32 hold the two column halves
    // of a row in a wave; the WGN waves of a row are merged through LDS in
    // wave order. (The target logit is read back by the merge kernel.)
    __shared__ float xs[WGN][BM][2];
    static_assert(NS * kStage >= BM * BN * 2, "the stages must hold the staged bf16 tile");
    __syncthreads();   // every wave is past its last fragment read: the stages are free
    if (n0 + BN <= g.N)
      xent_tile_stats<TM, TN, true, BM, BN>(g, acc, xs[wn], smem, n0, n0 + wn * WTN, wm * WTM, lane);
    else
      xent_tile_stats<TM, TN, false, BM, BN>(g, acc, xs[wn], smem, n0, n0 + wn * WTN, wm * WTM, lane);
    __syncthreads();
    CStage<bf16, BN, NW * 64>::flush(smem, BM, g.C, g.ldc, m0, n0, g.M, g.N, (int)threadIdx.x);
    for (int rt = threadIdx.x; rt < BM; rt += NW * 64) {
      const int m = m0 + rt;
      if (m >= g.M) continue;
      float M = xs[0][rt][0], S = xs[0][rt][1];
#pragma unroll
      for (int w = 1; w < WGN; ++w) {
        const float m2 = xs[w][rt][0], s2 = xs[w][rt][1];
        const float mn = fmaxf(M, m2);
        if (mn != -INFINITY) {
          S = S * __expf(M - mn) + s2 * __expf(m2 - mn);
          M = mn;
        }
      }
      float* o = g.xpart + ((int64_t)(n0 / BN) * g.M + m) * 2;
      o[0] = M;
      o[1] = S;
    }
    return;
  }

  // epilogue through LDS (all four stages, once every wave is past its last
  // fragment read)
  using Stage = CStage<TC, BN, NW * 64>;
  static_assert(NS * kStage >= BM * Stage::kRowBytes, "the stages must hold the staged tile");
  // GeLU epilogue: round 0 stages GeLU'(u) and leaves GeLU(u) in the
  // accumulators, round 1 stages those
  constexpr int kRounds = EPI == EPI_BIAS_GELU ? 2 : 1;
  BiasCols<TN> bias;
  if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) bias.load(g.bias, g.N, n0 + wn * WTN, lane);
  __syncthreads();
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rt = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nt = wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if constexpr (EPI == EPI_BIAS) bias.add(v, j, q);
          if constexpr (EPI == EPI_BIAS_GELU) {
            if (round == 0) {
              bias.add(v, j, q);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float ge, gp;
                gelu_and_grad(v[e], ge, gp);
                acc[i][j][4 * q + e] = ge;
                v[e] = gp;
              }
            }
          }
          Stage::put4(smem, rt, nt, v);
        }
      }
    }
    __syncthreads();
    Stage::flush(smem, BM, round == 0 ? g.C : g.C2, round == 0 ? g.ldc : g.ldc2, m0, n0, g.M, g.N,
                 (int)threadIdx.x);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ split-K sum
// C[m][n] += ws[0][m][n] + ws[1][m][n] + ... in split order (deterministic).
__global__ __launch_bounds__(256) void splitk_sum_kernel(float* C, int64_t ldc, const float* __restrict__ ws,
                                                         int nsum, int M, int N) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)M * N) return;
  const int64_t m = i / N, n = i % N;
  float* c = C + m * ldc + n;
  f32x4 acc = *reinterpret_cast<const f32x4*>(c);
  for (int sp = 0; sp < nsum; ++sp) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ws + (int64_t)sp * M * N + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  *reinterpret_cast<f32x4*>(c) = acc;
}

// The work after a paired launch, one role per workgroup: a split
// activation gradient's slices summed in split order and rounded to bf16
// (workgroups [0, red_blocks)), the weight gradient's split slices added into
// its output (the next sum_blocks), then the pair's column-sum tail.
struct TailArgs {
  int kind, nblk;
  ColFinal f;
  ColPartBf16 p;
  bf16* rc;             // split activation gradient: output, row stride, slices, count, shape
  int64_t ldrc;
  const float* rws;
  int rsplits, rM, rN, red_blocks;
};
__global__ __launch_bounds__(256) void splitk_sum_tail_kernel(float* C, int64_t ldc, const float* __restrict__ ws,
                                                              int nsum, int M, int N, int sum_blocks, TailArgs t) {
  if ((int)blockIdx.x < t.red_blocks) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (int64_t)t.rM * t.rN) return;
    const int64_t m = i / t.rN, n = i % t.rN;
    f32x4 acc = *reinterpret_cast<const f32x4*>(t.rws + i);
    for (int sp = 1; sp < t.rsplits; ++sp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(t.rws + (int64_t)sp * t.rM * t.rN + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    store4(t.rc + m * t.ldrc + n, acc[0], acc[1], acc[2], acc[3]);
    return;
  }
  const int bid = (int)blockIdx.x - t.red_blocks;
  if (bid < sum_blocks) {
    const int64_t i = ((int64_t)bid * 256 + threadIdx.x) * 4;
    if (i >= (int64_t)M * N) return;
    const int64_t m = i / N, n = i % N;
    float* c = C + m * ldc + n;
    f32x4 acc = *reinterpret_cast<const f32x4*>(c);
    for (int sp = 0; sp < nsum; ++sp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(ws + (int64_t)sp * M * N + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    *reinterpret_cast<f32x4*>(c) = acc;
    return;
  }
  const int b = bid - sum_blocks;
  if (t.kind == TAIL_COLSUM_FINAL) col_final(t.f, b);
  else colpart_bf16_block(t.p, b);
}

struct SplitK { int splits, kchunk, tile; };

// C[m][n] = ws[0][m][n] + ws[1][m][n] + ... in split order, stored as TC.
template <typename TC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(TC* C, int64_t ldc, const float* __restrict__ ws,
                                                            int nsplit, int M, int N) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)M * N) return;
  const int64_t m = i / N, n = i % N;
  f32x4 acc = *reinterpret_cast<const f32x4*>(ws + i);
  for (int sp = 1; sp < nsplit; ++sp) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ws + (int64_t)sp * M * N + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  if constexpr (sizeof(TC) == 2) {
    store4(C + m * ldc + n, acc[0], acc[1], acc[2], acc[3]);
  } else {
    *reinterpret_cast<f32x4*>(C + m * ldc + n) = acc;
  }
}

// Split of a bf16 data-gradient product (A K-major, B MN-major) whose
// 256x256 grid is small and whose K is long (the loss's dH over the
// vocabulary): every split writes fp32 partials into the workspace, summed
// and rounded once afterwards. Bounded by the workspace capacity.
int device_cus();

SplitK splitk_dgrad_for(int dtype, int64_t M, int64_t N, int64_t K, size_t ws_floats) {
  SplitK r{1, (int)K, 0};
  if (dtype != DT_BF16 || getenv("TPL_GEMM_TILE") || M * N <= 0) return r;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= 384) return r;
  const int64_t cus = device_cus();
  int64_t sp = 0;
  if (K >= 8192) {
    // 256x256 tiles: about one round of splits at least 4096 deep (the loss's
    // dH at 8192 x 1024 over 51200: 2 splits, 25-40 us faster than 4 splits in
    // two rounds, with half the partials to add); when K is too short for
    // that to fill the round (the output projection of a wide rank: 48
    // tiles, K = 12288), one round of splits at least 2048 deep
    sp = std::min<int64_t>((256 + tiles - 1) / tiles, K / 4096);
    if (tiles * sp < cus) sp = std::min<int64_t>(cus / tiles, K / 2048);
    r.tile = 256;
  } else {
    // 128x128 tiles (two workgroups per CU) filling under half their slots
    // (the output projection of a narrow rank: 96 tiles, K = 3072): splits at
    // least 1024 deep up to about one round
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (t128 * 2 >= 2 * cus || K < 2048) return r;
    sp = std::min<int64_t>(2 * cus / t128, K / 1024);
    r.tile = 128;
  }
  sp = std::min<int64_t>(sp, (int64_t)(ws_floats / (size_t)(M * N)));
  if (sp < 2) return SplitK{1, (int)K, 0};
  const int64_t chunk = ((K + sp - 1) / sp + 63) / 64 * 64;
  r.splits = (int)((K + chunk - 1) / chunk);
  r.kchunk = (int)chunk;
  return r;
}

// Compute units of the current device (cached per device).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  static std::atomic<int> cache[64];
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Split of a weight-gradient product (both operands MN-major, fp32 output)
// whose 256x256 grid is under a round of the CUs: the 256x256 tile with
// enough splits for about one round (each at least 1024 deep in K, and at
// least three quarters of the CUs busy), else the 128x128 tile with enough
// splits for about two workgroups per CU (each at least 1024 deep). Split 0
// writes C, the others the workspace, summed into C in split order. tile = 0:
// no split.
SplitK splitk_for(int dtype, int64_t M, int64_t N, int64_t K) {
  SplitK r{1, (int)K, 0};
  if (dtype != DT_BF16 || getenv("TPL_GEMM_TILE")) return r;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 384 || t256 == 0) return r;   // 256x256 tile, enough workgroups
  const int cus = device_cus();
  int64_t sp = std::min<int64_t>(cus / t256, K / 1024);
  int tile = 256;
  if (sp < 2 || 4 * t256 * sp < 3 * cus) {
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    sp = std::min<int64_t>(K / 1024, 512 / std::max<int64_t>(tiles, 1));
    tile = 128;
  }
  if (sp < 2) return r;
  const int64_t chunk = ((K + sp - 1) / sp + 63) / 64 * 64;
  r.splits = (int)((K + chunk - 1) / chunk);
  r.kchunk = (int)chunk;
  r.tile = tile;
  return r;
}

// Tail split of an fp32-output product on the 256x256 one-workgroup-per-CU
// tile. When its tiles fill the CUs for r whole rounds and leave a short last
// round (at most half the CUs busy for a whole tile's time), the tile rows of
// that round run first instead, split over K so that they occupy the chip for
// a fraction of a tile's time. Their fp32 partials live in the output rows
// that the whole rounds write afterwards (no extra memory), and are summed in
// split order (deterministic) into the tail rows before those rounds run.
// row0 = first tail row (M when no split).
struct TailSplit { int64_t row0; int splits, kchunk; };
TailSplit tail_split_for(int64_t M, int64_t N, int64_t K, int cus) {
  TailSplit t{M, 1, (int)K};
  if (getenv("TPL_GEMM_TILE") || getenv("TPL_GEMM_NO_TAIL_SPLIT")) return t;
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, nblk = tm * tn;
  if (nblk < cus) return t;
  const int64_t rows_dp = (nblk / cus) * cus / tn;   // whole tile rows of the whole rounds
  const int64_t tail = (tm - rows_dp) * tn;
  if (tail == 0 || 2 * tail > cus) return t;
  const int64_t tail_m = M - rows_dp * 256;
  int64_t sp = std::min<int64_t>(cus / tail, K / 512);
  sp = std::min<int64_t>(sp, rows_dp * 256 / tail_m);   // every partial fits in the rows written later
  if (sp < 2) return t;
  const int64_t chunk = ((K + sp - 1) / sp + 63) / 64 * 64;
  t.row0 = rows_dp * 256;
  t.splits = (int)((K + chunk - 1) / chunk);
  t.kchunk = (int)chunk;
  return t;
}

// A weight-gradient product with between one and one and a half rounds of
// 256x256 tiles would take three rounds of the 128x128 tile (two per CU,
// relative per-CU throughput 0.8); the 256x256 tile with the tail split takes
// its whole round plus the split tail rows (time of each in units of one
// full-depth 256x256 round). Only for K >= 4096: measured on the 8.3B rank's
// dE (300 tiles, K = 4096) 198 -> 182 us, but on the 175B rank's dW_o (288
// tiles, K = 2048) 106 -> 110 us.
bool tail_beats_128(int64_t M, int64_t N, int64_t K, const TailSplit& t, int cus) {
  if (K < 4096) return false;
  const int64_t tn = (N + 255) / 256, whole = (t.row0 / 256) * tn;
  const int64_t tail = ((M - t.row0 + 255) / 256) * tn;
  const double r256 = (double)((whole + cus - 1) / cus) +
                      (double)((tail * t.splits + cus - 1) / cus) * (double)t.kchunk / (double)K;
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const double r128 = (double)((t128 + 2 * cus - 1) / (2 * cus)) * (128.0 * 128.0 * 2.0 / 0.8) / 65536.0;
  return r256 < r128;
}

// ------------------------------------------------------------------ dispatch

struct TileCfg { int bm, bn, variant; };



template <typename T, int BM, int BN, int WM, int WN, bool AK, bool BK_, int EPI, typename TC>
hipError_t run(const GemmDesc& d, hipStream_t s) {
  Args a{};
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

// Tile choice. Forward products with at least 1024 tiles of 256x256 (the
// logits) take the four-stage 32-deep K pipeline. Other forward (NT) and
// activation-gradient (NN) products take the candidate with the least
//   rounds x (tile area x workgroups per CU) / throughput,
// rounds = ceil(tiles / (workgroups per CU x CUs)): a partly filled last round
// costs a whole one. Relative per-CU throughputs, fitted to timings of every
// forward and gradient product of the four bf16 layer shards on MI355X:
// 256x256 (8 waves, one workgroup per CU) 1.0; 256x192 (forward only) 0.8;
// 256x128 (forward only, 8 waves as 4 x 2) 0.75; 128x128 (4 waves, two per
// CU) 0.7 forward, 0.8 gradient. (256x128 won some gradient products timed
// alone but lost inside the layer pass, where the operands arrive from the
// previous kernels instead of a warm cache. In the layer pass the model
// gives it the forward products whose 256x256 grid is about half a round:
// 8.3B rank fc1 (192 tiles) 68 -> 55 us and QKV 44 -> 42 us, GPT-2 fc2 (256
// tiles) 79 -> 67 us and output projection 25 -> 24 us.) The
// 256x256 tile runs as 2 x 4 waves of 128x64 for forward products and 4 x 2
// waves of 64x128 for gradient products (faster there by up to 14% in the
// same timings). Weight-gradient (TN) products keep 256x256 with 2 x 4 waves
// when that gives at least 384 workgroups, else 128x128 (the split-K and
// tail-split paths decide their own tiles).
// TPL_GEMM_TILE=256x256[w8[t]] | 256x128[w8[t]] | 128x128 | 256x256w8s4 |
// 256x192w8t forces a shape (the tests use it to cover every tile path).
TileCfg choose_tile(int dtype, bool ak, bool bk, int64_t M, int64_t N, int epi = EPI_NONE) {
  const bool nt = ak && bk;
  if (dtype == DT_F32) return {128, 128, 0};
  if (const char* f = getenv("TPL_GEMM_TILE")) {
    if (!strcmp(f, "256x256")) return {256, 256, 0};
    if (!strcmp(f, "256x256w8")) return {256, 256, 1};
    if (!strcmp(f, "256x256w8t")) return {256, 256, 2};
    if (!strcmp(f, "256x128")) return {256, 128, 0};
    if (!strcmp(f, "256x128w8")) return {256, 128, 3};
    if (!strcmp(f, "256x128w8t")) return {256, 128, 4};
    if (!strcmp(f, "128x128")) return {128, 128, 0};
    if (!strcmp(f, "256x256w8s4")) return {256, 256, nt ? 5 : 1};
    if (!strcmp(f, "256x192w8t")) return nt ? TileCfg{256, 192, 6} : TileCfg{256, 256, 2};
  }
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  if (!ak && !bk) return big >= 384 ? TileCfg{256, 256, 1} : TileCfg{128, 128, 0};
  if (nt && big >= 1024) return {256, 256, 5};
  struct Cand { TileCfg t; int per_cu; double thr; };
  const int64_t cus = device_cus();
  (void)epi;
  Cand cands[4];
  int nc = 0;
  if (nt) {
    cands[nc++] = {{256, 256, 1}, 1, 1.0};
    cands[nc++] = {{256, 192, 6}, 1, 0.8};
    cands[nc++] = {{128, 128, 0}, 2, 0.7};
    cands[nc++] = {{256, 128, 4}, 1, 0.75};
  } else {
    cands[nc++] = {{256, 256, 2}, 1, 1.0};
    cands[nc++] = {{128, 128, 0}, 2, 0.8};
  }
  TileCfg best = cands[0].t;
  double best_cost = 0.0;
  for (int i = 0; i < nc; ++i) {
    const Cand& c = cands[i];
    const int64_t tiles = ((M + c.t.bm - 1) / c.t.bm) * ((N + c.t.bn - 1) / c.t.bn);
    const int64_t rounds = (tiles + c.per_cu * cus - 1) / (c.per_cu * cus);
    const double cost = (double)rounds * c.t.bm * c.t.bn * c.per_cu / c.thr;
    if (i == 0 || cost < best_cost) {
      best = c.t;
      best_cost = cost;
    }
  }
  return best;
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BK_, int EPI, typename TC>
hipError_t run_v2(const GemmDesc& d, hipStream_t s) {
  constexpr bool kDma = AK && BK_;   // LDS-DMA for the forward products, register staging otherwise
  Args a{};
  a.A = static_cast<const char*>(d.A); a.lda = d.lda;
  a.B = static_cast<const char*>(d.B); a.ldb = d.ldb;
  a.C = static_cast<char*>(d.C); a.ldc = d.ldc;
  a.C2 = static_cast<char*>(d.C2); a.ldc2 = d.ldc2;
  a.bias = static_cast<const char*>(d.bias);
  a.M = (int)d.M; a.N = (int)d.N; a.K = (int)d.K;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.splits = 1;
  a.kchunk = a.K;
  a.ws = nullptr;
  a.colpart = EPI == EPI_DGELU ? d.colpart : nullptr;
  if (!AK && !BK_ && d.c_f32 && d.ws && BM == BN) {
    const SplitK sk = splitk_for(d.dtype, d.M, d.N, d.K);
    if (sk.tile == BM) {
      a.splits = sk.splits;
      a.kchunk = sk.kchunk;
      a.ws = d.ws;
    }
  }
  const int nblk = a.tiles_m * a.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, AK, BK_, kDma, EPI, TC>), dim3(nblk * a.splits),
                     dim3(WGM * WGN * 64), 0, s, a);
  if (a.splits > 1) {
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const int64_t quads = (d.M * d.N + 3) / 4;
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s,
                       static_cast<float*>(d.C), d.ldc, d.ws, a.splits - 1, a.M, a.N);
  }
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int NS, int OCC, int EPI, typename TC>
hipError_t run_ms(const GemmDesc& d, hipStream_t s) {
  Args a{};
  a.A = static_cast<const char*>(d.A); a.lda = d.lda;
  a.B = static_cast<const char*>(d.B); a.ldb = d.ldb;
  a.C = static_cast<char*>(d.C); a.ldc = d.ldc;
  a.C2 = static_cast<char*>(d.C2); a.ldc2 = d.ldc2;
  a.bias = static_cast<const char*>(d.bias);
  a.M = (int)d.M; a.N = (int)d.N; a.K = (int)d.K;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.targets = d.targets; a.v0 = d.v0; a.xpart = d.xpart;
  const int nblk = a.tiles_m * a.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_ms_kernel<BM, BN, WGM, WGN, NS, OCC, EPI, TC>), dim3(nblk), dim3(WGM * WGN * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, bool AK, bool BK_, int EPI, typename TC>
hipError_t run_tiles(const GemmDesc& d, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    return run<T, 128, 128, 2, 2, AK, BK_, EPI, TC>(d, s);
  } else {
    const TileCfg t = choose_tile(d.dtype, AK, BK_, d.M, d.N, EPI);
    switch (t.variant) {
      case 1: return run_v2<256, 256, 2, 4, AK, BK_, EPI, TC>(d, s);
      case 2: return run_v2<256, 256, 4, 2, AK, BK_, EPI, TC>(d, s);
      case 3: return run_v2<256, 128, 2, 4, AK, BK_, EPI, TC>(d, s);
      case 4: return run_v2<256, 128, 4, 2, AK, BK_, EPI, TC>(d, s);
      case 5:
        if constexpr (AK && BK_) return run_ms<256, 256, 2, 4, 4, 2, EPI, TC>(d, s);
        break;
      case 6:   // forward products only (the MN-major layouts assume power-of-two tile widths)
        if constexpr (AK && BK_) return run_v2<256, 192, 4, 2, AK, BK_, EPI, TC>(d, s);
        break;
      default: break;
    }
    if (t.bm == 256 && t.bn == 256) return run_v2<256, 256, 2, 2, AK, BK_, EPI, TC>(d, s);
    if (t.bm == 256 && t.bn == 128) return run_v2<256, 128, 2, 2, AK, BK_, EPI, TC>(d, s);
    return run_v2<128, 128, 2, 2, AK, BK_, EPI, TC>(d, s);
  }
}

// bf16 dgrad split over K: the 256x256 8-wave (or 128x128 4-wave) kernel
// writes every split's fp32 partial into the workspace (C = ws, splits s >= 1 at ws + s*M*N), then
// one pass sums them in split order and rounds to bf16.
hipError_t run_dgrad_split(const GemmDesc& d, const SplitK& sk, hipStream_t s) {
  Args a{};
  a.A = static_cast<const char*>(d.A); a.lda = d.lda;
  a.B = static_cast<const char*>(d.B); a.ldb = d.ldb;
  a.C = reinterpret_cast<char*>(d.ws); a.ldc = d.N;
  a.C2 = nullptr; a.ldc2 = 0;
  a.bias = nullptr;
  a.M = (int)d.M; a.N = (int)d.N; a.K = (int)d.K;
  const int bt = sk.tile == 128 ? 128 : 256;
  a.tiles_m = (a.M + bt - 1) / bt;
  a.tiles_n = (a.N + bt - 1) / bt;
  a.targets = nullptr; a.v0 = 0; a.xpart = nullptr;
  a.splits = sk.splits;
  a.kchunk = sk.kchunk;
  a.ws = d.ws + (int64_t)d.M * d.N;
  const int nblk = a.tiles_m * a.tiles_n;
  if (bt == 128)
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, true, false, false, EPI_NONE, float>),
                       dim3(nblk * a.splits), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 4, true, false, false, EPI_NONE, float>),
                       dim3(nblk * a.splits), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t quads = (d.M * d.N + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s,
                     static_cast<bf16*>(d.C), d.ldc, static_cast<const float*>(d.ws), a.splits, a.M, a.N);
  return hipGetLastError();
}

// Weight-gradient product (both operands MN-major, fp32 output, ldc == N)
// with a tail split: the K-split pass over rows [row0, M) writes its partials
// into C rows [0, splits*(M-row0)), the sum fills rows [row0, M), then the
// whole rounds write rows [0, row0).
hipError_t run_tn_tail(const GemmDesc& d, const TailSplit& t, hipStream_t s) {
  const int64_t tail_m = d.M - t.row0;
  Args a{};
  a.A = static_cast<const char*>(d.A) + t.row0 * 2; a.lda = d.lda;
  a.a_trim = t.row0 * 2;   // the view starts row0 columns in: its last row ends row0 columns early
  a.B = static_cast<const char*>(d.B); a.ldb = d.ldb;
  a.C = static_cast<char*>(d.C); a.ldc = d.N;
  a.M = (int)tail_m; a.N = (int)d.N; a.K = (int)d.K;
  a.tiles_m = (a.M + 255) / 256;
  a.tiles_n = (a.N + 255) / 256;
  a.splits = t.splits;
  a.kchunk = t.kchunk;
  a.ws = static_cast<float*>(d.C) + tail_m * d.N;
  hipLaunchKernelGGL((gemm_bf16_tail_kernel<256, 256, 2, 4, false, false, false, EPI_NONE, float>),
                     dim3(a.tiles_m * a.tiles_n * a.splits), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t quads = (tail_m * d.N + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s,
                     static_cast<float*>(d.C) + t.row0 * d.ldc, d.ldc, static_cast<const float*>(d.C), t.splits,
                     (int)tail_m, (int)d.N);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmDesc w = d;
  w.M = t.row0;
  return run_v2<256, 256, 2, 4, false, false, EPI_NONE, float>(w, s);
}

// Arguments of one product of a paired launch (256x256 tiles, no split).
Args pair_args(const GemmDesc& d, int tile = 256) {
  Args a{};
  a.A = static_cast<const char*>(d.A); a.lda = d.lda;
  a.B = static_cast<const char*>(d.B); a.ldb = d.ldb;
  a.C = static_cast<char*>(d.C); a.ldc = d.ldc;
  a.C2 = static_cast<char*>(d.C2); a.ldc2 = d.ldc2;
  a.bias = static_cast<const char*>(d.bias);
  a.M = (int)d.M; a.N = (int)d.N; a.K = (int)d.K;
  a.tiles_m = (a.M + tile - 1) / tile;
  a.tiles_n = (a.N + tile - 1) / tile;
  a.splits = 1;
  a.kchunk = a.K;
  a.ws = nullptr;
  a.colpart = d.epi == EPI_DGELU ? d.colpart : nullptr;
  return a;
}

// Makespan (in units of one 256x256 tile step of depth 1) of list scheduling
// tiles on `cus` compute units in grid order: groups of (count, depth K).
double list_makespan(const int64_t (*groups)[2], int ngroups, int cus) {
  std::vector<double> free_at((size_t)cus, 0.0);
  std::make_heap(free_at.begin(), free_at.end(), std::greater<double>());
  double end = 0.0;
  for (int g = 0; g < ngroups; ++g) {
    for (int64_t i = 0; i < groups[g][0]; ++i) {
      std::pop_heap(free_at.begin(), free_at.end(), std::greater<double>());
      const double t = free_at.back() + (double)groups[g][1];
      free_at.back() = t;
      std::push_heap(free_at.begin(), free_at.end(), std::greater<double>());
      end = std::max(end, t);
    }
  }
  return end;
}

template <typename T>
hipError_t dispatch(const GemmDesc& d, hipStream_t s) {
  if (d.a_kmajor && d.b_kmajor) {
    if (d.c_f32) return hipErrorInvalidValue;
    switch (d.epi) {
      case EPI_NONE: return run_tiles<T, true, true, EPI_NONE, T>(d, s);
      case EPI_BIAS: return run_tiles<T, true, true, EPI_BIAS, T>(d, s);
      case EPI_BIAS_GELU: return run_tiles<T, true, true, EPI_BIAS_GELU, T>(d, s);
      case EPI_XENT:
        if constexpr (sizeof(T) == 2) {
          if (xent_gemm_tile_cols(d.dtype, d.M, d.N) == (int)((d.N + 255) / 256))
            return run_ms<256, 256, 2, 4, 4, 2, EPI_XENT, T>(d, s);
          return run_ms<128, 128, 2, 2, 4, 2, EPI_XENT, T>(d, s);
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
  if (d.a_kmajor && !d.b_kmajor) {
    if (d.c_f32) return hipErrorInvalidValue;
    if constexpr (sizeof(T) == 2) {
      if (d.epi == EPI_NONE && d.ws) {
        const SplitK sk = splitk_dgrad_for(d.dtype, d.M, d.N, d.K, d.ws_floats);
        if (sk.splits > 1) return run_dgrad_split(d, sk, s);
      }
    }
    switch (d.epi) {
      case EPI_NONE: return run_tiles<T, true, false, EPI_NONE, T>(d, s);
      case EPI_DGELU: return run_tiles<T, true, false, EPI_DGELU, T>(d, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (!d.a_kmajor && !d.b_kmajor && d.c_f32 && d.epi == EPI_NONE) {
    if constexpr (sizeof(T) == 2) {
      if (d.ws && splitk_for(d.dtype, d.M, d.N, d.K).tile == 256)
        return run_v2<256, 256, 2, 4, false, false, EPI_NONE, float>(d, s);
      if (d.ldc == d.N) {
        const TailSplit t = tail_split_for(d.M, d.N, d.K, device_cus());
        if (t.splits > 1 && (choose_tile(d.dtype, false, false, d.M, d.N).variant == 1 ||
                             tail_beats_128(d.M, d.N, d.K, t, device_cus())))
          return run_tn_tail(d, t, s);
      }
    }
    return run_tiles<T, false, false, EPI_NONE, float>(d, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// The fused-statistics logits product takes the 256x256 four-stage tile or
// its 128x128 form (two workgroups per CU), by the forward products' cost
// model: rounds over the CUs x tile area x workgroups per CU / throughput
// (1.0 and 0.7), a partly filled round costing a whole one.
int xent_gemm_tile_cols(int dtype, int64_t M, int64_t N) {
  if (dtype != DT_BF16 || M <= 0 || N <= 0) return 0;
  const int64_t cus = device_cus();
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256), t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const double c256 = (double)((t256 + cus - 1) / cus) * 65536.0;
  const double c128 = (double)((t128 + 2 * cus - 1) / (2 * cus)) * 32768.0 / 0.7;
  return c256 <= c128 ? (int)((N + 255) / 256) : (int)((N + 127) / 128);
}
size_t gemm_dgrad_ws_floats(int dtype, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 0;
  const SplitK sk = splitk_dgrad_for(dtype, M, N, K, ~size_t(0));
  return sk.splits > 1 ? (size_t)sk.splits * (size_t)M * (size_t)N : 0;
}
size_t gemm_ws_floats(int dtype, int64_t M, int64_t N, int64_t K) {
  const SplitK sk = splitk_for(dtype, M, N, K);
  return sk.splits > 1 ? (size_t)(sk.splits - 1) * (size_t)M * (size_t)N : 0;
}
int64_t gemm_colpart_chunks(int dtype, int64_t M, int64_t N) {
  if (dtype != DT_BF16) return 0;   // the fp32 kernel takes no column partials
  const TileCfg t = choose_tile(dtype, true, false, M, N, EPI_DGELU);
  const int nt = (t.variant >= 1 && t.variant <= 4) ? 512 : 256;   // threads of the chosen workgroup
  const int rc = t.bm / (nt / t.bn);                                  // rows per partial block
  return (M + rc - 1) / rc;
}
// Pairing of a block's activation-gradient product dg (A K-major, B
// MN-major, bf16 out, EPI_NONE or EPI_DGELU) with its weight-gradient product
// wg (both MN-major, fp32 out, ldc == N) in one grid of 256x256 tiles (or,
// for a dg without an epilogue, 128x128 tiles where that schedules better). Either
// may be split over K inside the grid: wg's splits >= 1 write fp32 slices
// summed into its output in split order afterwards; an EPI_NONE dg split
// writes all its splits as fp32 slices, summed in split order and rounded
// once into its output. The plan takes the pair of splits (each at least 1024
// deep) whose list schedule of both tile sets on the CUs (longer tiles first)
// ends soonest, and is chosen when that beats the two products launched
// apart (each split over K as it would be alone; wg unsplit counted as
// perfectly packed, which its tail split approaches). Times: a 256x256 tile
// of depth K takes 2*256*256*K flops at ~4.3 TFLOP/s per CU (the measured
// per-CU rate of these kernels), and every fp32 slice costs its write and read
// back at ~5 TB/s. TPL_GEMM_PAIR=0/1 forces the choice and
// TPL_GEMM_PAIR_TILE=256/128 the tile (tests). Workspace:
// dg's column partials (EPI_DGELU) or its split slices, then wg's slices.
namespace {

constexpr double kTileSecPerK = 2.0 * 256 * 256 / 4.3e12;
constexpr double kSliceSecPerFloat = 8.0 / 5.0e12;

// Splits of depth K each at least 1024 deep, as the kernels cut them
// (chunk rounded up to 64); 0 when sp does not come out exactly.
int64_t pair_chunk(int64_t K, int sp) {
  if (sp > 1 && K / sp < 1024) return 0;
  const int64_t chunk = ((K + sp - 1) / sp + 63) / 64 * 64;
  return (K + chunk - 1) / chunk == sp ? chunk : 0;
}

PairPlan plan_pair(const GemmDesc& dg, const GemmDesc& wg, bool* wanted) {
  PairPlan p{1, (int)dg.K, 1, (int)wg.K};
  *wanted = false;
  if (dg.dtype != DT_BF16 || wg.dtype != DT_BF16) return p;
  if (!dg.a_kmajor || dg.b_kmajor || dg.c_f32 || (dg.epi != EPI_NONE && dg.epi != EPI_DGELU)) return p;
  if (wg.a_kmajor || wg.b_kmajor || !wg.c_f32 || wg.epi != EPI_NONE || wg.ldc != wg.N) return p;
  if (dg.M <= 0 || dg.N <= 0 || dg.K <= 0 || wg.M <= 0 || wg.N <= 0 || wg.K <= 0) return p;
  const char* force = getenv("TPL_GEMM_PAIR");
  if (!force && getenv("TPL_GEMM_TILE")) return p;
  const int cus = device_cus();
  const int64_t td = ((dg.M + 255) / 256) * ((dg.N + 255) / 256), tw = ((wg.M + 255) / 256) * ((wg.N + 255) / 256);
  const double dmn = (double)dg.M * (double)dg.N, wmn = (double)wg.M * (double)wg.N;
  double best = 0.0;
  bool first = true;
  for (int sd = 1; sd <= (dg.epi == EPI_NONE ? 8 : 1); ++sd) {
    const int64_t cd = pair_chunk(dg.K, sd);
    if (!cd) continue;
    for (int sw = 1; sw <= 8; ++sw) {
      const int64_t cw = pair_chunk(wg.K, sw);
      if (!cw) continue;
      int64_t groups[2][2] = {{td * sd, cd}, {tw * sw, cw}};
      if (cw > cd) {
        std::swap(groups[0][0], groups[1][0]);
        std::swap(groups[0][1], groups[1][1]);
      }
      const double t = list_makespan(groups, 2, cus) * kTileSecPerK +
                       (sd > 1 ? (double)sd * dmn * kSliceSecPerFloat : 0.0) +
                       (double)(sw - 1) * wmn * kSliceSecPerFloat;
      if (first || t < best) {
        first = false;
        best = t;
        p = PairPlan{sd, (int)cd, sw, (int)cw};
      }
    }
  }
  // the same search on 128x128 tiles (activation gradients without an
  // epilogue): two workgroups per CU, each at 0.8 of the 256x256 tile's
  // per-CU rate, so a 128x128 tile of depth K takes 0.625 K units on one of
  // 2 * cus slots
  const char* ft = getenv("TPL_GEMM_PAIR_TILE");
  const int tile_force = ft ? atoi(ft) : 0;
  if (dg.epi == EPI_NONE && tile_force != 256) {
    const int64_t td1 = ((dg.M + 127) / 128) * ((dg.N + 127) / 128), tw1 = ((wg.M + 127) / 128) * ((wg.N + 127) / 128);
    bool first1 = true;
    double best1 = 0.0;
    PairPlan p1 = p;
    for (int sd = 1; sd <= 8; ++sd) {
      const int64_t cd = pair_chunk(dg.K, sd);
      if (!cd) continue;
      for (int sw = 1; sw <= 8; ++sw) {
        const int64_t cw = pair_chunk(wg.K, sw);
        if (!cw) continue;
        int64_t groups[2][2] = {{td1 * sd, cd}, {tw1 * sw, cw}};
        if (cw > cd) {
          std::swap(groups[0][0], groups[1][0]);
          std::swap(groups[0][1], groups[1][1]);
        }
        const double t = list_makespan(groups, 2, 2 * cus) * 0.625 * kTileSecPerK +
                         (sd > 1 ? (double)sd * dmn * kSliceSecPerFloat : 0.0) +
                         (double)(sw - 1) * wmn * kSliceSecPerFloat;
        if (first1 || t < best1) {
          first1 = false;
          best1 = t;
          p1 = PairPlan{sd, (int)cd, sw, (int)cw, 128};
        }
      }
    }
    if (!first1 && (tile_force == 128 || best1 < best)) {
      best = best1;
      p = p1;
    }
  }
  if (force) {
    *wanted = force[0] == '1';
    return p;
  }
  // apart: dg on its own rounds (or its own split over K), then wg
  double apart = 0.0;
  const SplitK skd = dg.epi == EPI_NONE ? splitk_dgrad_for(dg.dtype, dg.M, dg.N, dg.K, ~size_t(0)) : SplitK{1, 0, 0};
  // a 128x128 workgroup has a quarter of the 256x256 work, two per CU, at
  // 0.8 of the 256x256 tile's per-CU rate (the tile cost model's figure)
  auto split_time = [&](const SplitK& sk, int64_t M, int64_t N, int64_t t256) {
    const int64_t tiles = sk.tile == 128 ? ((M + 127) / 128) * ((N + 127) / 128) : t256;
    const int64_t w[1][2] = {{tiles * sk.splits, sk.kchunk}};
    return (sk.tile == 128 ? list_makespan(w, 1, 2 * cus) / 4.0 * 2.0 / 0.8 : list_makespan(w, 1, cus)) * kTileSecPerK;
  };
  if (skd.splits > 1) {
    apart += split_time(skd, dg.M, dg.N, td) + (double)skd.splits * dmn * kSliceSecPerFloat;
  } else {
    const int64_t one[1][2] = {{td, dg.K}};
    apart += list_makespan(one, 1, cus) * kTileSecPerK;
  }
  const SplitK sk = splitk_for(wg.dtype, wg.M, wg.N, wg.K);
  if (sk.splits > 1) {
    apart += split_time(sk, wg.M, wg.N, tw) + (double)(sk.splits - 1) * wmn * kSliceSecPerFloat;
  } else if (choose_tile(wg.dtype, false, false, wg.M, wg.N).bm == 128) {
    apart += split_time(SplitK{1, (int)wg.K, 128}, wg.M, wg.N, tw);
  } else {
    apart += (double)tw * (double)wg.K / cus * kTileSecPerK;
  }
  // measured: the pair wins even where the model puts it a few percent short
  // of the two launches (8.3B rank fc1 backward, model 100.7 vs 104.7 us:
  // 117.6 -> 107.1 us), so any modelled gain takes it
  *wanted = best < apart;
  return p;
}

}  // namespace

// Plans are memoized per (shapes, epilogue, CU count, forcing variables):
// the search list-schedules up to 64 split pairs and costs up to ~0.25 ms of
// host time, and every backward call asks for its plans twice (workspace
// size, launch).
bool gemm_pair_plan(const GemmDesc& dg, const GemmDesc& wg, PairPlan* plan) {
  struct Key {
    int64_t v[10];
    bool operator==(const Key& o) const { return std::equal(v, v + 10, o.v); }
  };
  struct Entry { Key k; PairPlan p; bool wanted; };
  static std::mutex mu;
  static std::vector<Entry> memo;
  const char* force = getenv("TPL_GEMM_PAIR");
  const char* ftile = getenv("TPL_GEMM_PAIR_TILE");
  const int64_t fk = (force ? (force[0] == '1' ? 2 : 1) : (getenv("TPL_GEMM_TILE") ? 3 : 0)) +
                     4 * (ftile ? (int64_t)atoi(ftile) : 0);
  const int64_t flags = (dg.a_kmajor ? 1 : 0) | (dg.b_kmajor ? 2 : 0) | (dg.c_f32 ? 4 : 0) | (wg.a_kmajor ? 8 : 0) |
                        (wg.b_kmajor ? 16 : 0) | (wg.c_f32 ? 32 : 0) | (int64_t)(wg.ldc == wg.N) << 6 |
                        (int64_t)dg.dtype << 8 | (int64_t)wg.dtype << 12 | (int64_t)dg.epi << 16 |
                        (int64_t)wg.epi << 20 | fk << 24;
  const Key k{{dg.M, dg.N, dg.K, wg.M, wg.N, wg.K, flags, (int64_t)device_cus(), 0, 0}};
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : memo)
      if (e.k == k) {
        *plan = e.p;
        return e.wanted;
      }
  }
  bool wanted = false;
  *plan = plan_pair(dg, wg, &wanted);
  std::lock_guard<std::mutex> lock(mu);
  if (memo.size() >= 256) memo.clear();
  memo.push_back(Entry{k, *plan, wanted});
  return wanted;
}

// Column-partial blocks the paired activation-gradient product writes for
// EPI_DGELU (128 rows each: the 256x256 tile's eight waves as 4 x 2).
int64_t gemm_pair_colpart_chunks(int64_t M) { return (M + 127) / 128; }

namespace {
// Workspace of a pair: dg's column partials (EPI_DGELU) or split slices,
// padded to 64 floats, then wg's slices.
size_t pair_dg_floats(const GemmDesc& dg, const PairPlan& plan) {
  size_t f = 0;
  if (dg.epi == EPI_DGELU) f = (size_t)gemm_pair_colpart_chunks(dg.M) * (size_t)dg.N;
  else if (plan.dg_splits > 1) f = (size_t)plan.dg_splits * (size_t)dg.M * (size_t)dg.N;
  return (f + 63) / 64 * 64;
}
}  // namespace

size_t gemm_pair_ws_floats(const GemmDesc& dg, const GemmDesc& wg, const PairPlan& plan) {
  return pair_dg_floats(dg, plan) + (size_t)(plan.wg_splits - 1) * (size_t)wg.M * (size_t)wg.N;
}

hipError_t launch_gemm_pair(const GemmDesc& dg, const GemmDesc& wg, const PairPlan& plan, float* ws,
                            hipStream_t s, const PairTail* tail) {
  TraceScope trace(K_GEMM_PAIR, s, 2.0 * (double)dg.M * dg.N * dg.K + 2.0 * (double)wg.M * wg.N * wg.K);
  if (dg.dtype != DT_BF16 || wg.dtype != DT_BF16 || plan.wg_splits < 1 || plan.dg_splits < 1) return hipErrorInvalidValue;
  if (plan.dg_splits > 1 && dg.epi != EPI_NONE) return hipErrorInvalidValue;
  if ((plan.wg_splits > 1 || plan.dg_splits > 1 || dg.epi == EPI_DGELU) && !ws) return hipErrorInvalidValue;
  if (plan.tile != 256 && (plan.tile != 128 || dg.epi != EPI_NONE)) return hipErrorInvalidValue;
  Args a0 = pair_args(dg, plan.tile), a1 = pair_args(wg, plan.tile);
  a0.colpart = dg.epi == EPI_DGELU ? ws : nullptr;
  const bool dsplit = plan.dg_splits > 1;
  if (dsplit) {   // every split of dg into fp32 slices: slice 0 at ws, slice s at ws + s*M*N
    a0.C = reinterpret_cast<char*>(ws);
    a0.ldc = dg.N;
    a0.splits = plan.dg_splits;
    a0.kchunk = plan.dg_kchunk;
    a0.ws = ws + (int64_t)dg.M * dg.N;
  }
  if (plan.wg_splits > 1) {
    a1.splits = plan.wg_splits;
    a1.kchunk = plan.wg_kchunk;
    a1.ws = ws + pair_dg_floats(dg, plan);
  }
  const int64_t t0 = (int64_t)a0.tiles_m * a0.tiles_n * a0.splits, t1 = (int64_t)a1.tiles_m * a1.tiles_n * a1.splits;
  if (t0 + t1 + 8 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const bool wg_first = a1.kchunk > a0.kchunk;   // the longer tiles start first
  const int n0 = (int)(wg_first ? t1 : t0), n0pad = (n0 + 7) / 8 * 8, n1 = (int)(wg_first ? t0 : t1);
  if (n0 + n1 == 0) return hipSuccess;
  const dim3 grid((unsigned)(n0pad + n1)), block(plan.tile == 128 ? 256 : 512);
  if (plan.tile == 128) {
    if (dsplit) {
      if (wg_first)
        hipLaunchKernelGGL((gemm_pair128_kernel<false, false, float, true, false, float>), grid, block, 0, s, a1, a0, n0,
                           n0pad);
      else
        hipLaunchKernelGGL((gemm_pair128_kernel<true, false, float, false, false, float>), grid, block, 0, s, a0, a1, n0,
                           n0pad);
    } else if (wg_first) {
      hipLaunchKernelGGL((gemm_pair128_kernel<false, false, float, true, false, bf16>), grid, block, 0, s, a1, a0, n0,
                         n0pad);
    } else {
      hipLaunchKernelGGL((gemm_pair128_kernel<true, false, bf16, false, false, float>), grid, block, 0, s, a0, a1, n0,
                         n0pad);
    }
  } else if (dsplit) {   // both products on the 2 x 4 wave layout with fp32 output
    if (wg_first)
      hipLaunchKernelGGL((gemm_pair_kernel<2, 4, false, false, EPI_NONE, float, 2, 4, true, false, EPI_NONE, float>),
                         grid, block, 0, s, a1, a0, n0, n0pad);
    else
      hipLaunchKernelGGL((gemm_pair_kernel<2, 4, true, false, EPI_NONE, float, 2, 4, false, false, EPI_NONE, float>),
                         grid, block, 0, s, a0, a1, n0, n0pad);
  } else if (wg_first) {
    if (dg.epi == EPI_DGELU)
      hipLaunchKernelGGL((gemm_pair_kernel<2, 4, false, false, EPI_NONE, float, 4, 2, true, false, EPI_DGELU, bf16>),
                         grid, block, 0, s, a1, a0, n0, n0pad);
    else
      hipLaunchKernelGGL((gemm_pair_kernel<2, 4, false, false, EPI_NONE, float, 4, 2, true, false, EPI_NONE, bf16>),
                         grid, block, 0, s, a1, a0, n0, n0pad);
  } else {
    if (dg.epi == EPI_DGELU)
      hipLaunchKernelGGL((gemm_pair_kernel<4, 2, true, false, EPI_DGELU, bf16, 2, 4, false, false, EPI_NONE, float>),
                         grid, block, 0, s, a0, a1, n0, n0pad);
    else
      hipLaunchKernelGGL((gemm_pair_kernel<4, 2, true, false, EPI_NONE, bf16, 2, 4, false, false, EPI_NONE, float>),
                         grid, block, 0, s, a0, a1, n0, n0pad);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TailArgs t{};
  if (dsplit) {   // dg's slices summed and rounded in the same launch as wg's sum and the tail
    t.rc = static_cast<bf16*>(dg.C);
    t.ldrc = dg.ldc;
    t.rws = ws;
    t.rsplits = plan.dg_splits;
    t.rM = a0.M;
    t.rN = a0.N;
    t.red_blocks = (int)(((dg.M * dg.N + 3) / 4 + 255) / 256);
  }
  t.kind = tail ? tail->kind : TAIL_NONE;
  if (t.kind == TAIL_COLSUM_FINAL) {
    t.f = ColFinal{tail->ws, {tail->out, nullptr, nullptr}, (int)tail->nchunks, 1, tail->cols, 0};
    t.nblk = col_final_blocks(1, tail->cols);
  } else if (t.kind == TAIL_COLSUM_PARTIALS) {
    const int nbx = (tail->cols / 8 + 63) / 64;
    t.p = ColPartBf16{static_cast<const bf16*>(tail->X), tail->ld, tail->rows, tail->cols, nbx, 0, tail->ws};
    t.nblk = nbx * (int)((tail->rows + kRowsPerChunk - 1) / kRowsPerChunk);
  } else if (t.kind != TAIL_NONE) {
    return hipErrorInvalidValue;
  }
  const int64_t quads = plan.wg_splits > 1 ? (wg.M * wg.N + 3) / 4 : 0;
  const int sum_blocks = (int)((quads + 255) / 256);
  if (t.red_blocks + sum_blocks + t.nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_sum_tail_kernel, dim3((unsigned)(t.red_blocks + sum_blocks + t.nblk)), dim3(256), 0, s,
                     static_cast<float*>(wg.C), wg.ldc, a1.ws, plan.wg_splits - 1, a1.M, a1.N, sum_blocks, t);
  return hipGetLastError();
}

size_t xent_part_floats(int64_t M, int64_t N) { return (size_t)((N + 127) / 128) * (size_t)M * 2; }

int device_cu_count() { return device_cus(); }

hipError_t launch_gemm(const GemmDesc& d, hipStream_t s) {
  TraceScope trace(d.a_kmajor && d.b_kmajor ? K_GEMM_NT : (d.a_kmajor ? K_GEMM_NN : K_GEMM_TN), s,
                   2.0 * (double)d.M * (double)d.N * (double)d.K);
  if (d.dtype == DT_BF16) return dispatch<bf16>(d, s);
  return dispatch<float>(d, s);
}

}  // namespace tpl
