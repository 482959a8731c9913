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
// deterministic stages (per row-chunk partials, then a fixed-order sum).
#include "common.h"
#include "kernels.h"

namespace tpl {
namespace {

constexpr int kRowsPerChunk = 64;

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& raw, float* v) {
  Vec16<T> x;
  x.raw = raw;
#pragma unroll
  for (int e = 0; e < Vec16<T>::N; ++e) v[e] = to_f32(x.get(e));
}
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
  u32x4 cache[MAXC];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + 64 * i;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (ch < nch) raw = ld16(xr + ch * V);
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
      unpack<T>(ld16(g + ch * V), gv);
      unpack<T>(ld16(bta + ch * V), bv);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
      st16(yr + ch * V, pack<T>(v));
    }
  }
  if (lane == 0) { mu_out[row] = mean; rstd_out[row] = rstd; }
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

// Column partials for LN backward: ws[chunk][0][c] = sum dsum*xhat,
// ws[chunk][1][c] = sum dsum, ws[chunk][2][c] = sum dy over the chunk's rows.
template <typename T>
__global__ __launch_bounds__(64) void ln_bwd_cols_kernel(const T* __restrict__ dy, const T* __restrict__ dsum,
                                                         const T* __restrict__ x, const float* __restrict__ mu,
                                                         const float* __restrict__ rstd, float* __restrict__ ws,
                                                         int64_t rows, int cols) {
  constexpr int V = Vec16<T>::N;
  const int ch = blockIdx.x * 64 + threadIdx.x;
  if (ch * V >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * kRowsPerChunk;
  const int64_t r1 = min<int64_t>(rows, r0 + kRowsPerChunk);
  float a[V], b[V], c[V];
#pragma unroll
  for (int e = 0; e < V; ++e) { a[e] = 0.f; b[e] = 0.f; c[e] = 0.f; }
  for (int64_t r = r0; r < r1; ++r) {
    float dv[V], xv[V], yv[V];
    unpack<T>(ld16(dsum + r * cols + ch * V), dv);
    unpack<T>(ld16(x + r * cols + ch * V), xv);
    unpack<T>(ld16(dy + r * cols + ch * V), yv);
    const float m = mu[r], rs = rstd[r];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      a[e] += dv[e] * (xv[e] - m) * rs;
      b[e] += dv[e];
      c[e] += yv[e];
    }
  }
  float* w = ws + (int64_t)blockIdx.y * 3 * cols + ch * V;
#pragma unroll
  for (int e = 0; e < V; ++e) { w[e] = a[e]; w[cols + e] = b[e]; w[2 * cols + e] = c[e]; }
}

// Column partials of one matrix: ws[chunk][c] = sum over the chunk's rows of X[r][c].
template <typename T>
__global__ __launch_bounds__(64) void colsum_kernel(const T* __restrict__ X, int64_t ld, int64_t rows,
                                                    int cols, float* __restrict__ ws) {
  constexpr int V = Vec16<T>::N;
  const int ch = blockIdx.x * 64 + threadIdx.x;
  if (ch * V >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * kRowsPerChunk;
  const int64_t r1 = min<int64_t>(rows, r0 + kRowsPerChunk);
  float a[V];
#pragma unroll
  for (int e = 0; e < V; ++e) a[e] = 0.f;
  for (int64_t r = r0; r < r1; ++r) {
    float v[V];
    unpack<T>(ld16(X + r * ld + ch * V), v);
#pragma unroll
    for (int e = 0; e < V; ++e) a[e] += v[e];
  }
  float* w = ws + (int64_t)blockIdx.y * cols + ch * V;
#pragma unroll
  for (int e = 0; e < V; ++e) w[e] = a[e];
}

// out_k[c] = sum over chunks of ws[chunk][k][c], for k < nout. One block of
// 4 waves per 64 columns: wave w sums chunks w, w+4, ... (lane = column), the
// four wave sums are then added in wave order -- a fixed order, so the result
// is deterministic.
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ ws, int nchunks, int cols,
                                                           int nout, float* o0, float* o1, float* o2) {
  __shared__ float part[3][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  for (int k = 0; k < nout; ++k) {
    float s0 = 0.f, s1 = 0.f;
    if (c < cols) {
      int i = wave;
      for (; i + 4 < nchunks; i += 8) {
        s0 += ws[((int64_t)i * nout + k) * cols + c];
        s1 += ws[((int64_t)(i + 4) * nout + k) * cols + c];
      }
      if (i < nchunks) s0 += ws[((int64_t)i * nout + k) * cols + c];
    }
    part[k][wave][lane] = s0 + s1;
  }
  __syncthreads();
  if (wave == 0 && c < cols) {
    float* outs[3] = {o0, o1, o2};
    for (int k = 0; k < nout; ++k)
      outs[k][c] = (part[k][0][lane] + part[k][1][lane]) + (part[k][2][lane] + part[k][3][lane]);
  }
}

// ------------------------------------------------------------------ partial sum
struct PartPtrs { const void* p[16]; };

template <typename T>
__global__ __launch_bounds__(256) void partial_sum_kernel(PartPtrs parts, int n, const T* __restrict__ bias,
                                                          const T* __restrict__ residual, T* out,
                                                          int64_t rows, int cols) {
  constexpr int V = Vec16<T>::N;
  const int64_t nvec = rows * (cols / V);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  const int64_t row = i / (cols / V);
  const int col = (int)(i % (cols / V)) * V;
  const int64_t off = row * cols + col;
  float acc[V], t[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  if (residual) {
    unpack<T>(ld16(residual + off), t);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] += t[e];
  }
  if (bias) {
    unpack<T>(ld16(bias + col), t);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] += t[e];
  }
  for (int k = 0; k < n; ++k) {
    unpack<T>(ld16(static_cast<const T*>(parts.p[k]) + off), t);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] += t[e];
  }
  st16(out + off, pack<T>(acc));
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

#define TPL_MAXC_SWITCH(M, CALL)      \
  switch (M) {                        \
    case 1: { constexpr int MC = 1; return CALL; }  \
    case 2: { constexpr int MC = 2; return CALL; }  \
    case 4: { constexpr int MC = 4; return CALL; }  \
    case 8: { constexpr int MC = 8; return CALL; }  \
    case 16: { constexpr int MC = 16; return CALL; } \
    case 24: { constexpr int MC = 24; return CALL; } \
    case 32: { constexpr int MC = 32; return CALL; } \
  }                                   \
  return hipErrorInvalidValue;

int64_t n_chunks(int64_t rows) { return (rows + kRowsPerChunk - 1) / kRowsPerChunk; }

}  // namespace

size_t layernorm_bwd_ws_floats(int64_t rows, int cols) { return (size_t)n_chunks(rows) * 3 * cols; }
size_t colsum_ws_floats(int64_t rows, int cols) { return (size_t)n_chunks(rows) * cols; }

hipError_t launch_layernorm_fwd(int dtype, const void* x, const void* g, const void* b, void* y, float* mu,
                                float* rstd, int64_t rows, int cols, float eps, hipStream_t s) {
  TraceScope trace(K_LN_FWD, s, (double)rows * cols * 2 * dtype_size(dtype) + rows * 8.0);
  const int mc = maxc_for(dtype, cols);
  if (dtype == DT_BF16) { TPL_MAXC_SWITCH(mc, (ln_fwd_t<bf16, MC>(x, g, b, y, mu, rstd, rows, cols, eps, s))) }
  TPL_MAXC_SWITCH(mc, (ln_fwd_t<float, MC>(x, g, b, y, mu, rstd, rows, cols, eps, s)))
}

static hipError_t ln_bwd_rows(int dtype, const void* dy, const void* dsum, const void* x, const float* mu,
                              const float* rstd, const void* g, void* dx, int64_t rows, int cols, hipStream_t s) {
  TraceScope trace(K_LN_BWD, s, (double)rows * cols * 4 * dtype_size(dtype) + rows * 8.0);
  const int mc = maxc_for(dtype, cols);
  if (dtype == DT_BF16) { TPL_MAXC_SWITCH(mc, (ln_bwd_t<bf16, MC>(dy, dsum, x, mu, rstd, g, dx, rows, cols, s))) }
  TPL_MAXC_SWITCH(mc, (ln_bwd_t<float, MC>(dy, dsum, x, mu, rstd, g, dx, rows, cols, s)))
}

hipError_t launch_layernorm_bwd(int dtype, const void* dy, const void* dsum, const void* x, const float* mu,
                                const float* rstd, const void* g, void* dx, float* d_g, float* d_b,
                                float* d_bout, float* ws, int64_t rows, int cols, hipStream_t s) {
  hipError_t e;
  {
    TraceScope trace(K_LN_BWD_COLS, s, (double)rows * cols * 3 * dtype_size(dtype));
    const int v = dtype == DT_BF16 ? 8 : 4;
    dim3 grid((cols / v + 63) / 64, (unsigned)n_chunks(rows));
    if (dtype == DT_BF16)
      hipLaunchKernelGGL(ln_bwd_cols_kernel<bf16>, grid, dim3(64), 0, s, static_cast<const bf16*>(dy),
                         static_cast<const bf16*>(dsum), static_cast<const bf16*>(x), mu, rstd, ws, rows, cols);
    else
      hipLaunchKernelGGL(ln_bwd_cols_kernel<float>, grid, dim3(64), 0, s, static_cast<const float*>(dy),
                         static_cast<const float*>(dsum), static_cast<const float*>(x), mu, rstd, ws, rows, cols);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    TraceScope trace(K_COLSUM_FINAL, s);
    hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 63) / 64), dim3(256), 0, s, ws, (int)n_chunks(rows), cols,
                       3, d_g, d_b, d_bout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // rows last: dx may alias dy (the residual path is read before it is overwritten per row)
  return ln_bwd_rows(dtype, dy, dsum, x, mu, rstd, g, dx, rows, cols, s);
}

hipError_t launch_colsum(int dtype, const void* X, int64_t ld, int64_t rows, int cols, float* out, float* ws,
                         hipStream_t s) {
  hipError_t e;
  {
    TraceScope trace(K_COLSUM, s, (double)rows * cols * dtype_size(dtype));
    const int v = dtype == DT_BF16 ? 8 : 4;
    dim3 grid((cols / v + 63) / 64, (unsigned)n_chunks(rows));
    if (dtype == DT_BF16)
      hipLaunchKernelGGL(colsum_kernel<bf16>, grid, dim3(64), 0, s, static_cast<const bf16*>(X), ld, rows, cols, ws);
    else
      hipLaunchKernelGGL(colsum_kernel<float>, grid, dim3(64), 0, s, static_cast<const float*>(X), ld, rows, cols, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  TraceScope trace(K_COLSUM_FINAL, s);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 63) / 64), dim3(256), 0, s, ws, (int)n_chunks(rows), cols, 1,
                     out, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_partial_sum(int dtype, const void* const* parts, int n, const void* bias, const void* residual,
                              void* out, int64_t rows, int cols, hipStream_t s) {
  TraceScope trace(K_PARTIAL_SUM, s, (double)rows * cols * (n + 1 + (residual ? 1 : 0)) * dtype_size(dtype));
  PartPtrs pp;
  for (int i = 0; i < 16; ++i) pp.p[i] = i < n ? parts[i] : nullptr;
  const int v = dtype == DT_BF16 ? 8 : 4;
  const int64_t nvec = rows * (cols / v);
  const dim3 grid((unsigned)((nvec + 255) / 256));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(partial_sum_kernel<bf16>, grid, dim3(256), 0, s, pp, n, static_cast<const bf16*>(bias),
                       static_cast<const bf16*>(residual), static_cast<bf16*>(out), rows, cols);
  else
    hipLaunchKernelGGL(partial_sum_kernel<float>, grid, dim3(256), 0, s, pp, n, static_cast<const float*>(bias),
                       static_cast<const float*>(residual), static_cast<float*>(out), rows, cols);
  return hipGetLastError();
}

}  // namespace tpl
