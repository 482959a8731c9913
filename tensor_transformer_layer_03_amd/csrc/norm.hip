// Row and column kernels of the layer shard: LayerNorm forward/backward
// (replicated on every rank -- podcast page, Outline: dropout, LayerNorm and
// residual are duplicated rather than communicated), deterministic column
// sums for bias / LN-parameter gradients, and the all-reduce stand-in that
// adds the row-parallel partials, the bias and the residual (podcast page,
// Key concepts: all-reduce).
//
// All of these are HBM-bound: they stream each operand once with 16-byte
// vector accesses. LayerNorm uses one wave per row with the row cached in
// registers (two-pass mean / variance, no LDS); column sums run in two
// deterministic stages (per 32-row-chunk partials, then a fixed-order sum).
#include "colsum.h"
#include "common.h"
#include "kernels.h"

namespace tpl {
namespace {

template <typename T>
__device__ __forceinline__ u32x4 pack(const float* v) {
  Vec16<T> x;
#pragma unroll
  for (int e = 0; e < Vec16<T>::N; ++e) x.set(e, from_f32<T>(v[e]));
  return x.raw;
}

// ------------------------------------------------------------------ LayerNorm forward
// One wave per row; lane handles chunks c = lane + 64*i (16 B each), i < MAXC.
template <typename T, int MAXC>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                     const T* __restrict__ bta, T* __restrict__ y,
                                                     float* __restrict__ mu_out, float* __restrict__ rstd_out,
                                                     int64_t rows, int cols, float eps) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = cols / V;
  const T* xr = x + row * cols;
  u32x4 cache[MAXC], gcache[MAXC], bcache[MAXC];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {   // gamma and beta are loaded with the row, ahead of the reductions
    const int ch = lane + 64 * i;
    u32x4 raw = {0u, 0u, 0u, 0u}, rg = raw, rb = raw;
    if (ch < nch) {
      raw = ld16(xr + ch * V);
      rg = ld16(g + ch * V);
      rb = ld16(bta + ch * V);
    }
    gcache[i] = rg;
    bcache[i] = rb;
    cache[i] = raw;
    float v[V];
    unpack<T>(raw, v);
#pragma unroll
    for (int e = 0; e < V; ++e) sum += v[e];
  }
  const float mean = wave_sum(sum) / cols;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float v[V];
      unpack<T>(cache[i], v);
#pragma unroll
      for (int e = 0; e < V; ++e) { const float d = v[e] - mean; sq += d * d; }
    }
  }
  const float rstd = rsqrtf(wave_sum(sq) / cols + eps);
  T* yr = y + row * cols;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float v[V], gv[V], bv[V];
      unpack<T>(cache[i], v);
      unpack<T>(gcache[i], gv);
      unpack<T>(bcache[i], bv);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
      st16(yr + ch * V, pack<T>(v));
    }
  }
  if (lane == 0) { mu_out[row] = mean; rstd_out[row] = rstd; }
}

// ------------------------------------------------------------------ wide rows
// Rows wider than two 16-B chunks per lane (hidden > 1024 in bf16): one
// workgroup of four waves per row, thread t caching chunks t + 256 i (PER per
// thread), so a row streams with 4x the loads in flight and the register
// cache stays small. Row sums: each wave's sum, then the four added in wave
// order through LDS (deterministic).
__device__ __forceinline__ float block4_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T, int PER>
__global__ __launch_bounds__(256) void ln_fwd_wide_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                          const T* __restrict__ bta, T* __restrict__ y,
                                                          float* __restrict__ mu_out, float* __restrict__ rstd_out,
                                                          int cols, float eps) {
  constexpr int V = Vec16<T>::N;
  __shared__ float red[2][4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nch = cols / V;
  const T* xr = x + row * cols;
  u32x4 cache[PER];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + 256 * i;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (ch < nch) raw = ld16(xr + ch * V);
    cache[i] = raw;
    float v[V];
    unpack<T>(raw, v);
#pragma unroll
    for (int e = 0; e < V; ++e) sum += v[e];
  }
  const float mean = block4_sum(sum, red[0]) / cols;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (tid + 256 * i < nch) {
      float v[V];
      unpack<T>(cache[i], v);
#pragma unroll
      for (int e = 0; e < V; ++e) { const float d = v[e] - mean; sq += d * d; }
    }
  }
  const float rstd = rsqrtf(block4_sum(sq, red[1]) / cols + eps);
  T* yr = y + row * cols;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + 256 * i;
    if (ch < nch) {
      float v[V], gv[V], bv[V];
      unpack<T>(cache[i], v);
      unpack<T>(ld16(g + ch * V), gv);
      unpack<T>(ld16(bta + ch * V), bv);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
      st16(yr + ch * V, pack<T>(v));
    }
  }
  if (tid == 0) { mu_out[row] = mean; rstd_out[row] = rstd; }
}


// dx = dy + rstd * (gd - mean(gd) - xhat * mean(gd * xhat)),  gd = dsum * gamma
// (as ln_bwd_kernel below), one workgroup per row.
template <typename T, int PER>
__global__ __launch_bounds__(256) void ln_bwd_wide_kernel(const T* __restrict__ dy, const T* __restrict__ dsum,
                                                          const T* __restrict__ x, const float* __restrict__ mu,
                                                          const float* __restrict__ rstd, const T* __restrict__ g,
                                                          T* __restrict__ dx, int cols, ColFinal f) {
  constexpr int V = Vec16<T>::N;
  __shared__ float red[2][4];
  if ((int)blockIdx.x < f.nblk) {   // the first workgroups finish the column sums instead
    col_final(f, (int)blockIdx.x);
    return;
  }
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x - f.nblk;
  const int nch = cols / V;
  const float m = mu[row], rs = rstd[row];
  u32x4 cd[PER], cx[PER], cy[PER];
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + 256 * i;
    u32x4 rd = {0u, 0u, 0u, 0u}, rx = rd, ry = rd;
    if (ch < nch) {
      rd = ld16(dsum + row * cols + ch * V);
      rx = ld16(x + row * cols + ch * V);
      ry = ld16(dy + row * cols + ch * V);
      float dv[V], xv[V], gv[V];
      unpack<T>(rd, dv);
      unpack<T>(rx, xv);
      unpack<T>(ld16(g + ch * V), gv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float gd = dv[e] * gv[e];
        s1 += gd;
        s2 += gd * (xv[e] - m) * rs;
      }
    }
    cd[i] = rd;
    cx[i] = rx;
    cy[i] = ry;
  }
  const float mean1 = block4_sum(s1, red[0]) / cols, mean2 = block4_sum(s2, red[1]) / cols;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + 256 * i;
    if (ch < nch) {
      float dv[V], xv[V], gv[V], yv[V];
      unpack<T>(cd[i], dv);
      unpack<T>(cx[i], xv);
      unpack<T>(ld16(g + ch * V), gv);
      unpack<T>(cy[i], yv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (xv[e] - m) * rs;
        yv[e] += rs * (dv[e] * gv[e] - mean1 - xh * mean2);
      }
      st16(dx + row * cols + ch * V, pack<T>(yv));
    }
  }
}

// ------------------------------------------------------------------ LayerNorm backward (rows)
// dx = dy + rstd * (gd - mean(gd) - xhat * mean(gd * xhat)),  gd = dsum * gamma.
template <typename T, int MAXC>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ dsum,
                                                     const T* __restrict__ x, const float* __restrict__ mu,
                                                     const float* __restrict__ rstd, const T* __restrict__ g,
                                                     T* __restrict__ dx, int64_t rows, int cols) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = cols / V;
  const float m = mu[row], rs = rstd[row];
  u32x4 cd[MAXC], cx[MAXC];
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + 64 * i;
    u32x4 rd = {0u, 0u, 0u, 0u}, rx = {0u, 0u, 0u, 0u};
    if (ch < nch) {
      rd = ld16(dsum + row * cols + ch * V);
      rx = ld16(x + row * cols + ch * V);
      float dv[V], xv[V], gv[V];
      unpack<T>(rd, dv);
      unpack<T>(rx, xv);
      unpack<T>(ld16(g + ch * V), gv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float gd = dv[e] * gv[e];
        s1 += gd;
        s2 += gd * (xv[e] - m) * rs;
      }
    }
    cd[i] = rd;
    cx[i] = rx;
  }
  const float mean1 = wave_sum(s1) / cols, mean2 = wave_sum(s2) / cols;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float dv[V], xv[V], gv[V], yv[V];
      unpack<T>(cd[i], dv);
      unpack<T>(cx[i], xv);
      unpack<T>(ld16(g + ch * V), gv);
      unpack<T>(ld16(dy + row * cols + ch * V), yv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (xv[e] - m) * rs;
        yv[e] += rs * (dv[e] * gv[e] - mean1 - xh * mean2);
      }
      st16(dx + row * cols + ch * V, pack<T>(yv));
    }
  }
}

// LayerNorm backward in one pass for rows of at most two 16-B chunks per lane
// (hidden <= 1024 in bf16): a workgroup of eight waves takes one chunk of
// kRowsPerChunk rows (wave w: rows w, w+8, w+16, w+24), loads all of its
// rows' dsum, x and dy at once, writes dx for them (as ln_bwd_kernel) and the
// chunk's column partials ws[chunk][k][c] (k = 0: sum of dsum * xhat, 1: sum
// of dsum, 2: sum of dy, each wave over its rows in order, then the eight
// wave sums in a fixed tree through LDS). One read of the three row tensors
// instead of two.
template <typename T>
__global__ __launch_bounds__(512) void ln_bwd_fused_kernel(const T* dy, const T* __restrict__ dsum,
                                                           const T* __restrict__ x, const float* __restrict__ mu,
                                                           const float* __restrict__ rstd, const T* __restrict__ g,
                                                           T* dx, float* __restrict__ ws, int64_t rows, int cols) {
  constexpr int V = Vec16<T>::N, MAXC = 2, NW = 8, RPW = kRowsPerChunk / NW;
  constexpr int kCols = 64 * MAXC * V;   // column slots of a workgroup
  __shared__ float part[NW][3][kCols];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerChunk;
  const int nch = cols / V;

  u32x4 rd[RPW][MAXC], rx[RPW][MAXC], ry[RPW][MAXC];
  float m[RPW], rs[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int64_t row = r0 + wave + NW * j;
    const bool live = row < rows;
    m[j] = live ? mu[row] : 0.f;
    rs[j] = live ? rstd[row] : 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int ch = lane + 64 * i;
      rd[j][i] = rx[j][i] = ry[j][i] = u32x4{0u, 0u, 0u, 0u};
      if (live && ch < nch) {
        rd[j][i] = ld16(dsum + row * cols + ch * V);
        rx[j][i] = ld16(x + row * cols + ch * V);
        ry[j][i] = ld16(dy + row * cols + ch * V);
      }
    }
  }
  float gv[MAXC][V];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) unpack<T>(ld16(g + ch * V), gv[i]);
    else
#pragma unroll
      for (int e = 0; e < V; ++e) gv[i][e] = 0.f;
  }
  float a[3][MAXC][V];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
#pragma unroll
      for (int e = 0; e < V; ++e) a[k][i][e] = 0.f;

#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int64_t row = r0 + wave + NW * j;
    if (row >= rows) break;   // uniform over the wave
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      float dv[V], xv[V], yv[V];
      unpack<T>(rd[j][i], dv);
      unpack<T>(rx[j][i], xv);
      unpack<T>(ry[j][i], yv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float gd = dv[e] * gv[i][e];
        s1 += gd;
        s2 += gd * (xv[e] - m[j]) * rs[j];
        a[0][i][e] += dv[e] * (xv[e] - m[j]) * rs[j];
        a[1][i][e] += dv[e];
        a[2][i][e] += yv[e];
      }
    }
    const float mean1 = wave_sum(s1) / cols, mean2 = wave_sum(s2) / cols;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) {
        float dv[V], xv[V], yv[V];
        unpack<T>(rd[j][i], dv);
        unpack<T>(rx[j][i], xv);
        unpack<T>(ry[j][i], yv);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float xh = (xv[e] - m[j]) * rs[j];
          yv[e] += rs[j] * (dv[e] * gv[i][e] - mean1 - xh * mean2);
        }
        st16(dx + row * cols + ch * V, pack<T>(yv));
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
#pragma unroll
      for (int e = 0; e < V; ++e) part[wave][k][(i * V + e) * 64 + lane] = a[k][i][e];
  __syncthreads();
  // slot q = (i*V + e)*64 + l holds column (l + 64 i)*V + e
  for (int idx = threadIdx.x; idx < 3 * kCols; idx += 64 * NW) {
    const int k = idx / kCols, q = idx % kCols;
    const int l = q % 64, ie = q / 64, i = ie / V, e = ie % V;
    const int c = (l + 64 * i) * V + e;
    if (c < cols)
      ws[((int64_t)blockIdx.x * 3 + k) * cols + c] =
          ((part[0][k][q] + part[1][k][q]) + (part[2][k][q] + part[3][k][q])) +
          ((part[4][k][q] + part[5][k][q]) + (part[6][k][q] + part[7][k][q]));
  }
}

template <typename T, int NOUT>
__global__ __launch_bounds__(256) void colpart_kernel(const T* __restrict__ X, int64_t ld,
                                                      const T* __restrict__ dy, const T* __restrict__ x,
                                                      const float* __restrict__ mu, const float* __restrict__ rstd,
                                                      float* __restrict__ ws, int64_t rows, int cols) {
  colpart_body<T, NOUT>(X, ld, dy, x, mu, rstd, ws, rows, cols, (int)blockIdx.x, (int)blockIdx.y);
}

// out_k[c] = sum over chunks of ws[chunk][k][c], for k < nout. One workgroup
// of 16 waves per 64 columns and output: wave w sums chunks w, w+16, ... with
// four accumulators (lane = column), then the sixteen wave sums are added in
// a fixed tree order, so the result is deterministic.
__global__ __launch_bounds__(1024) void colsum_final_kernel(const float* __restrict__ ws, int nchunks, int cols,
                                                            int nout, float* o0, float* o1, float* o2) {
  __shared__ float part[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int k = blockIdx.y;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  if (c < cols) {
    int i = wave;
    for (; i + 240 < nchunks; i += 256) {   // four rounds of loads in flight, added in round order
      float v[4][4];
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int u = 0; u < 4; ++u) v[it][u] = ws[((int64_t)(i + 64 * it + 16 * u) * nout + k) * cols + c];
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] += v[it][u];
    }
    for (; i + 48 < nchunks; i += 64) {
#pragma unroll
      for (int u = 0; u < 4; ++u) s[u] += ws[((int64_t)(i + 16 * u) * nout + k) * cols + c];
    }
    for (; i < nchunks; i += 16) s[0] += ws[((int64_t)i * nout + k) * cols + c];
  }
  part[wave][lane] = (s[0] + s[1]) + (s[2] + s[3]);
  __syncthreads();
  if (wave == 0 && c < cols) {
    float q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      q[u] = (part[4 * u][lane] + part[4 * u + 1][lane]) + (part[4 * u + 2][lane] + part[4 * u + 3][lane]);
    float* out = k == 0 ? o0 : (k == 1 ? o1 : o2);
    out[c] = (q[0] + q[1]) + (q[2] + q[3]);
  }
}

// ------------------------------------------------------------------ partial sum
struct PartPtrs { const void* p[16]; };

// The partial count NP is a template argument (one instantiation per count,
// 1..16), so a thread's loads occupy 4 NP registers per chunk instead of the
// 64 of a runtime count; each thread takes U chunks, 256 apart. bf16 takes
// U = 2: with eight partials of 4096 x 3072 a step's sums went 230 -> 215 us
// (447 -> 430 us at 2048 x 12288, four of 8192 x 2560 205 -> 193 us); U = 4
// was slower than 2 on all three.
template <typename T, int NP, int U>
__global__ __launch_bounds__(256) void partial_sum_kernel(PartPtrs parts, const T* __restrict__ bias,
                                                          const T* __restrict__ residual, T* out,
                                                          int64_t rows, int cols) {
  constexpr int V = Vec16<T>::N;
  const int cpr = cols / V;
  const int64_t nvec = rows * cpr;
  const int64_t i0 = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
  // every load is issued before the first add, then the values are added in
  // the fixed order residual, bias, partials 0..NP-1. The partials are read
  // once, with the non-temporal hint: eight partials of 4096 x 3072 took
  // 243 -> 230 us a step so, of 2048 x 12288 527 -> 445 us; the hint on the
  // store changed nothing.
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 rres[U], rbias[U], raw[U][NP];
  int64_t off[U];
  int col[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = i0 + 256 * u;
    const int64_t row = i / cpr;
    col[u] = (int)(i - row * cpr) * V;
    off[u] = row * cols + col[u];
    rres[u] = rbias[u] = zero;
    if (i < nvec) {
      if (residual) rres[u] = ld16(residual + off[u]);
      if (bias) rbias[u] = ld16(bias + col[u]);
#pragma unroll
      for (int k = 0; k < NP; ++k)
        raw[u][k] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const T*>(parts.p[k]) + off[u]));
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (i0 + 256 * u >= nvec) break;
    float acc[V], t[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;
    if (residual) {
      unpack<T>(rres[u], t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += t[e];
    }
    if (bias) {
      unpack<T>(rbias[u], t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += t[e];
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      unpack<T>(raw[u][k], t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += t[e];
    }
    st16(out + off[u], pack<T>(acc));
  }
}

template <typename T, int MAXC>
hipError_t ln_fwd_t(const void* x, const void* g, const void* b, void* y, float* mu, float* rstd, int64_t rows,
                    int cols, float eps, hipStream_t s) {
  hipLaunchKernelGGL((ln_fwd_kernel<T, MAXC>), dim3((rows + 3) / 4), dim3(256), 0, s,
                     static_cast<const T*>(x), static_cast<const T*>(g), static_cast<const T*>(b),
                     static_cast<T*>(y), mu, rstd, rows, cols, eps);
  return hipGetLastError();
}
template <typename T, int MAXC>
hipError_t ln_bwd_t(const void* dy, const void* dsum, const void* x, const float* mu, const float* rstd,
                    const void* g, void* dx, int64_t rows, int cols, hipStream_t s) {
  hipLaunchKernelGGL((ln_bwd_kernel<T, MAXC>), dim3((rows + 3) / 4), dim3(256), 0, s,
                     static_cast<const T*>(dy), static_cast<const T*>(dsum), static_cast<const T*>(x), mu, rstd,
                     static_cast<const T*>(g), static_cast<T*>(dx), rows, cols);
  return hipGetLastError();
}

// Register-cache depth: chunks of 16 B per lane, rounded up to a supported size.
int maxc_for(int dtype, int cols) {
  const int v = dtype == DT_BF16 ? 8 : 4;
  const int need = (cols / v + 63) / 64;
  const int sizes[] = {1, 2, 4, 8, 16, 24, 32};
  for (int m : sizes)
    if (need <= m) return m;
  return -1;
}

// wave-per-row kernels: at most two chunks per lane (wider rows take the
// one-workgroup-per-row kernels)
#define TPL_MAXC_SWITCH(M, CALL)      \
  switch (M) {                        \
    case 1: { constexpr int MC = 1; return CALL; }  \
    case 2: { constexpr int MC = 2; return CALL; }  \
  }                                   \
  return hipErrorInvalidValue;

int64_t n_chunks(int64_t rows) { return (rows + kRowsPerChunk - 1) / kRowsPerChunk; }

// Chunks per thread of the one-workgroup-per-row kernels (256 threads), or -1.
int wide_per(int dtype, int cols) {
  const int v = dtype == DT_BF16 ? 8 : 4;
  const int need = (cols / v + 255) / 256;
  const int sizes[] = {1, 2, 4, 8};
  for (int m : sizes)
    if (need <= m) return m;
  return -1;
}

#define TPL_PER_SWITCH(P, CALL)       \
  switch (P) {                        \
    case 1: { constexpr int PC = 1; return CALL; }  \
    case 2: { constexpr int PC = 2; return CALL; }  \
    case 4: { constexpr int PC = 4; return CALL; }  \
    case 8: { constexpr int PC = 8; return CALL; }  \
  }                                   \
  return hipErrorInvalidValue;

template <typename T, int PER>
hipError_t ln_fwd_wide_t(const void* x, const void* g, const void* b, void* y, float* mu, float* rstd, int64_t rows,
                         int cols, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((ln_fwd_wide_kernel<T, PER>), dim3((unsigned)rows), dim3(256), 0, s, static_cast<const T*>(x),
                     static_cast<const T*>(g), static_cast<const T*>(b), static_cast<T*>(y), mu, rstd, cols, eps);
  return hipGetLastError();
}
template <typename T, int PER>
hipError_t ln_bwd_wide_t(const void* dy, const void* dsum, const void* x, const float* mu, const float* rstd,
                         const void* g, void* dx, int64_t rows, int cols, const ColFinal& f, hipStream_t s) {
  if (rows + f.nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((ln_bwd_wide_kernel<T, PER>), dim3((unsigned)(rows + f.nblk)), dim3(256), 0, s,
                     static_cast<const T*>(dy), static_cast<const T*>(dsum), static_cast<const T*>(x), mu, rstd,
                     static_cast<const T*>(g), static_cast<T*>(dx), cols, f);
  return hipGetLastError();
}

}  // namespace

size_t layernorm_bwd_ws_floats(int64_t rows, int cols) { return (size_t)n_chunks(rows) * 3 * cols; }
size_t colsum_ws_floats(int64_t rows, int cols) { return (size_t)n_chunks(rows) * cols; }

hipError_t launch_layernorm_fwd(int dtype, const void* x, const void* g, const void* b, void* y, float* mu,
                                float* rstd, int64_t rows, int cols, float eps, hipStream_t s) {
  TraceScope trace(K_LN_FWD, s, (double)rows * cols * 2 * dtype_size(dtype) + rows * 8.0);
  const int mc = maxc_for(dtype, cols);
  if (mc > 2) {   // wide rows: one four-wave workgroup per row
    const int per = wide_per(dtype, cols);
    if (dtype == DT_BF16) { TPL_PER_SWITCH(per, (ln_fwd_wide_t<bf16, PC>(x, g, b, y, mu, rstd, rows, cols, eps, s))) }
    TPL_PER_SWITCH(per, (ln_fwd_wide_t<float, PC>(x, g, b, y, mu, rstd, rows, cols, eps, s)))
  }
  if (dtype == DT_BF16) { TPL_MAXC_SWITCH(mc, (ln_fwd_t<bf16, MC>(x, g, b, y, mu, rstd, rows, cols, eps, s))) }
  TPL_MAXC_SWITCH(mc, (ln_fwd_t<float, MC>(x, g, b, y, mu, rstd, rows, cols, eps, s)))
}

// Rows of the LayerNorm backward; on the wide-row path (one four-wave
// workgroup per row) the same launch also finishes the column sums f.
static hipError_t ln_bwd_rows(int dtype, const void* dy, const void* dsum, const void* x, const float* mu,
                              const float* rstd, const void* g, void* dx, int64_t rows, int cols, const ColFinal& f,
                              hipStream_t s) {
  TraceScope trace(K_LN_BWD, s, (double)rows * cols * 4 * dtype_size(dtype) + rows * 8.0);
  const int mc = maxc_for(dtype, cols);
  if (mc > 2) {   // wide rows: one four-wave workgroup per row
    const int per = wide_per(dtype, cols);
    if (dtype == DT_BF16) { TPL_PER_SWITCH(per, (ln_bwd_wide_t<bf16, PC>(dy, dsum, x, mu, rstd, g, dx, rows, cols, f, s))) }
    TPL_PER_SWITCH(per, (ln_bwd_wide_t<float, PC>(dy, dsum, x, mu, rstd, g, dx, rows, cols, f, s)))
  }
  if (f.nblk) return hipErrorInvalidValue;   // column sums ride only on the wide-row launch
  if (dtype == DT_BF16) { TPL_MAXC_SWITCH(mc, (ln_bwd_t<bf16, MC>(dy, dsum, x, mu, rstd, g, dx, rows, cols, s))) }
  TPL_MAXC_SWITCH(mc, (ln_bwd_t<float, MC>(dy, dsum, x, mu, rstd, g, dx, rows, cols, s)))
}

hipError_t launch_layernorm_bwd(int dtype, const void* dy, const void* dsum, const void* x, const float* mu,
                                const float* rstd, const void* g, void* dx, float* d_g, float* d_b,
                                float* d_bout, float* ws, int64_t rows, int cols, hipStream_t s) {
  hipError_t e;
  const int mc = maxc_for(dtype, cols);
  if (mc > 0 && mc <= 2) {   // rows and column partials in one pass
    {
      TraceScope trace(K_LN_BWD, s, (double)rows * cols * 4 * dtype_size(dtype) + rows * 8.0);
      const dim3 grid((unsigned)n_chunks(rows));
      if (dtype == DT_BF16)
        hipLaunchKernelGGL(ln_bwd_fused_kernel<bf16>, grid, dim3(512), 0, s, static_cast<const bf16*>(dy),
                           static_cast<const bf16*>(dsum), static_cast<const bf16*>(x), mu, rstd,
                           static_cast<const bf16*>(g), static_cast<bf16*>(dx), ws, rows, cols);
      else
        hipLaunchKernelGGL(ln_bwd_fused_kernel<float>, grid, dim3(512), 0, s, static_cast<const float*>(dy),
                           static_cast<const float*>(dsum), static_cast<const float*>(x), mu, rstd,
                           static_cast<const float*>(g), static_cast<float*>(dx), ws, rows, cols);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    TraceScope trace(K_COLSUM_FINAL, s);
    hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 63) / 64, 3), dim3(1024), 0, s, ws, (int)n_chunks(rows), cols,
                       3, d_g, d_b, d_bout);
    return hipGetLastError();
  }
  {
    TraceScope trace(K_LN_BWD_COLS, s, (double)rows * cols * 3 * dtype_size(dtype));
    const int v = dtype == DT_BF16 ? 8 : 4;
    dim3 grid((cols / v + 63) / 64, (unsigned)n_chunks(rows));
    if (dtype == DT_BF16)
      hipLaunchKernelGGL((colpart_kernel<bf16, 3>), grid, dim3(256), 0, s, static_cast<const bf16*>(dsum), (int64_t)cols,
                         static_cast<const bf16*>(dy), static_cast<const bf16*>(x), mu, rstd, ws, rows, cols);
    else
      hipLaunchKernelGGL((colpart_kernel<float, 3>), grid, dim3(256), 0, s, static_cast<const float*>(dsum),
                         (int64_t)cols, static_cast<const float*>(dy), static_cast<const float*>(x), mu, rstd, ws,
                         rows, cols);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  ColFinal f{ws, {d_g, d_b, d_bout}, (int)n_chunks(rows), 3, cols, 0};
  if (mc > 2) {
    // wide rows: the rows launch finishes the column sums in its first
    // workgroups (one launch fewer)
    f.nblk = col_final_blocks(3, cols);
  } else {
    TraceScope trace(K_COLSUM_FINAL, s);
    hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 63) / 64, 3), dim3(1024), 0, s, ws, (int)n_chunks(rows), cols,
                       3, d_g, d_b, d_bout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // rows last: dx may alias dy (the residual path is read before it is overwritten per row)
  return ln_bwd_rows(dtype, dy, dsum, x, mu, rstd, g, dx, rows, cols, f, s);
}

hipError_t launch_colsum(int dtype, const void* X, int64_t ld, int64_t rows, int cols, float* out, float* ws,
                         hipStream_t s) {
  hipError_t e;
  {
    TraceScope trace(K_COLSUM, s, (double)rows * cols * dtype_size(dtype));
    const int v = dtype == DT_BF16 ? 8 : 4;
    dim3 grid((cols / v + 63) / 64, (unsigned)n_chunks(rows));
    if (dtype == DT_BF16)
      hipLaunchKernelGGL((colpart_kernel<bf16, 1>), grid, dim3(256), 0, s, static_cast<const bf16*>(X), ld, nullptr,
                         nullptr, nullptr, nullptr, ws, rows, cols);
    else
      hipLaunchKernelGGL((colpart_kernel<float, 1>), grid, dim3(256), 0, s, static_cast<const float*>(X), ld, nullptr,
                         nullptr, nullptr, nullptr, ws, rows, cols);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  TraceScope trace(K_COLSUM_FINAL, s);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 63) / 64, 1), dim3(1024), 0, s, ws, (int)n_chunks(rows), cols, 1,
                     out, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_colsum_final(const float* ws, int64_t nchunks, int cols, float* out, hipStream_t s) {
  TraceScope trace(K_COLSUM_FINAL, s);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 63) / 64, 1), dim3(1024), 0, s, ws, (int)nchunks, cols, 1, out,
                     nullptr, nullptr);
  return hipGetLastError();
}

template <typename T, int U>
hipError_t launch_partial_sum_t(const PartPtrs& pp, int n, const void* bias, const void* residual, void* out,
                                int64_t rows, int cols, hipStream_t s) {
  const int64_t nvec = rows * (cols / Vec16<T>::N);
  const dim3 grid((unsigned)((nvec + 256 * U - 1) / (256 * U)));
  const T* b = static_cast<const T*>(bias);
  const T* r = static_cast<const T*>(residual);
  T* o = static_cast<T*>(out);
  switch (n) {
#define TPL_PSUM_CASE(NP) \
    case NP: hipLaunchKernelGGL((partial_sum_kernel<T, NP, U>), grid, dim3(256), 0, s, pp, b, r, o, rows, cols); break;
    TPL_PSUM_CASE(1) TPL_PSUM_CASE(2) TPL_PSUM_CASE(3) TPL_PSUM_CASE(4) TPL_PSUM_CASE(5) TPL_PSUM_CASE(6)
    TPL_PSUM_CASE(7) TPL_PSUM_CASE(8) TPL_PSUM_CASE(9) TPL_PSUM_CASE(10) TPL_PSUM_CASE(11) TPL_PSUM_CASE(12)
    TPL_PSUM_CASE(13) TPL_PSUM_CASE(14) TPL_PSUM_CASE(15) TPL_PSUM_CASE(16)
#undef TPL_PSUM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_partial_sum(int dtype, const void* const* parts, int n, const void* bias, const void* residual,
                              void* out, int64_t rows, int cols, hipStream_t s) {
  TraceScope trace(K_PARTIAL_SUM, s, (double)rows * cols * (n + 1 + (residual ? 1 : 0)) * dtype_size(dtype));
  if (n < 1 || n > 16) return hipErrorInvalidValue;
  PartPtrs pp;
  for (int i = 0; i < 16; ++i) pp.p[i] = i < n ? parts[i] : nullptr;
  if (dtype == DT_BF16) return launch_partial_sum_t<bf16, 2>(pp, n, bias, residual, out, rows, cols, s);
  return launch_partial_sum_t<float, 1>(pp, n, bias, residual, out, rows, cols, s);
}

}  // namespace tpl
