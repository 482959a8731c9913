// Deterministic column sums shared by the row kernels and the launches
// that follow the paired backward products: per-chunk column partials of a
// [rows][cols] operand and their fixed-order final sum. Device code only.
#pragma once
#include "common.h"

namespace tpl {
namespace {

constexpr int kRowsPerChunk = 32;

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& raw, float* v) {
  Vec16<T> x;
  x.raw = raw;
#pragma unroll
  for (int e = 0; e < Vec16<T>::N; ++e) v[e] = to_f32(x.get(e));
}

// Column partials. A workgroup covers 64 column chunks of 16 B and the
// kRowsPerChunk rows of one row chunk; wave w takes rows w, w+4, ... and the
// four wave sums are added in wave order through LDS, so every partial has a
// fixed summation order.
//   NOUT == 1: ws[chunk][0][c] = sum X[r][c]                       (bias gradients)
//   NOUT == 3: ws[chunk][0][c] = sum dsum*xhat, [1] = sum dsum, [2] = sum dy
//              (LN gamma / beta gradients and the next bias gradient)
template <typename T, int NOUT>
__device__ __forceinline__ void colpart_body(const T* __restrict__ X, int64_t ld, const T* __restrict__ dy,
                                             const T* __restrict__ x, const float* __restrict__ mu,
                                             const float* __restrict__ rstd, float* __restrict__ ws, int64_t rows,
                                             int cols, int bx, int by) {
  constexpr int V = Vec16<T>::N;
  __shared__ float part[4][NOUT][64 * V];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ch = bx * 64 + lane;
  const bool live = ch * V < cols;
  const int64_t r0 = (int64_t)by * kRowsPerChunk;
  const int64_t r1 = min<int64_t>(rows, r0 + kRowsPerChunk);
  float a[NOUT][V];
#pragma unroll
  for (int k = 0; k < NOUT; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) a[k][e] = 0.f;
  if (live) {
#pragma unroll 4
    for (int64_t r = r0 + wave; r < r1; r += 4) {
      float v[V];
      unpack<T>(ld16(X + r * ld + ch * V), v);   // NOUT == 3: X = dsum
      if constexpr (NOUT == 1) {
#pragma unroll
        for (int e = 0; e < V; ++e) a[0][e] += v[e];
      } else {
        float xv[V], yv[V];
        unpack<T>(ld16(x + r * ld + ch * V), xv);
        unpack<T>(ld16(dy + r * ld + ch * V), yv);
        const float m = mu[r], rs = rstd[r];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          a[0][e] += v[e] * (xv[e] - m) * rs;
          a[1][e] += v[e];
          a[2][e] += yv[e];
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NOUT; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) part[wave][k][e * 64 + lane] = a[k][e];
  __syncthreads();
  // 64*V columns x NOUT outputs, 256 threads: thread t finishes column slots t, t+256, ...
  const int64_t chunk = by;
  for (int idx = threadIdx.x; idx < NOUT * 64 * V; idx += 256) {
    const int k = idx / (64 * V), q = idx % (64 * V);
    const int e = q / 64, l = q % 64;
    const int c = (bx * 64 + l) * V + e;
    if (c < cols)
      ws[(chunk * NOUT + k) * cols + c] = (part[0][k][q] + part[1][k][q]) + (part[2][k][q] + part[3][k][q]);
  }
}

// Column sums finished inside another launch: out_k[c] = sum over chunks of
// ws[chunk][k][c] (the partials of colpart_kernel). Workgroup b (four waves)
// takes output k = b / ceil(cols / 64) and 64 consecutive columns (lane =
// column); wave w adds chunks w, w + 4, ... in ascending order into four
// accumulators, and the four wave sums are added in wave order: a fixed order.
struct ColFinal {
  const float* ws;
  float* out[3];
  int nchunks, nout, cols, nblk;   // nblk = 0: no column sums in this launch
};
constexpr int col_final_blocks(int nout, int cols) { return nout * ((cols + 63) / 64); }
__device__ __forceinline__ void col_final(const ColFinal& f, int b) {
  __shared__ float part[4][64];
  const int per_out = (f.cols + 63) / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = b / per_out, c = (b % per_out) * 64 + lane;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  if (c < f.cols) {
    const float* p = f.ws + (int64_t)k * f.cols + c;
    const int64_t step = (int64_t)f.nout * f.cols;
    int i = w;
    for (; i + 12 < f.nchunks; i += 16) {
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] += p[(int64_t)(i + 4 * u) * step];
    }
    for (; i < f.nchunks; i += 4) a[0] += p[(int64_t)i * step];
  }
  part[w][lane] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  if (w == 0 && c < f.cols) f.out[k][c] = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
}

// A [rows][cols] bf16 operand's NOUT == 1 column partials, one workgroup per
// (64 column chunks, row chunk), as a role inside another launch: nbx
// workgroups across the columns, blocks numbered column-block fastest.
struct ColPartBf16 {
  const bf16* X;
  int64_t ld, rows;
  int cols, nbx, nblk;
  float* ws;
};
__device__ __forceinline__ void colpart_bf16_block(const ColPartBf16& p, int b) {
  colpart_body<bf16, 1>(p.X, p.ld, nullptr, nullptr, nullptr, nullptr, p.ws, p.rows, p.cols, b % p.nbx, b / p.nbx);
}

}  // namespace
}  // namespace tpl
