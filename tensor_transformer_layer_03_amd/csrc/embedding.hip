// Vocabulary-parallel input embedding (guide page section 3.3: the input
// layer is split along the vocabulary and the ranks' outputs are summed by an
// all-reduce). Forward: this rank's masked lookup, zero rows for ids outside
// its range (the caller's partial sum then adds the ranks). Backward: the
// scatter-add of the output gradient into this rank's rows, made
// deterministic by a stable sort of (id, row) pairs: each vocabulary row then
// sums its gradient rows in ascending row order, with no atomics on floats.
//
// Memory-bound throughout: the lookup moves N*h elements twice; the gradient
// reads N*h elements once and writes the V_r*h fp32 table once (every row,
// zero where no id points).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace tpl {
namespace {

// out[n] = emb[tok[n] - v0] if 0 <= tok[n] - v0 < vr, else 0 (16-B chunks, flat).
template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* __restrict__ tok, const T* __restrict__ emb,
                                                        T* __restrict__ out, int64_t v0, int vr, int cpr,
                                                        uint32_t nchunks) {
  constexpr int V = Vec16<T>::N;
  const uint32_t c = blockIdx.x * 256u + threadIdx.x;
  if (c >= nchunks) return;
  const uint32_t n = c / (uint32_t)cpr, j = c - n * (uint32_t)cpr;
  const int64_t key = (int64_t)tok[n] - v0;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (key >= 0 && key < vr) v = ld16(emb + key * (int64_t)cpr * V + j * V);
  st16(out + (int64_t)c * V, v);
}

// keys[i] = tok[i] - v0 if in [0, vr) else vr (sorts last), vals[i] = i;
// seg[v] = -1 for every vocabulary row.
__global__ __launch_bounds__(256) void embed_keys_kernel(const int32_t* __restrict__ tok, int n, int64_t v0, int vr,
                                                         uint32_t* __restrict__ keys, uint32_t* __restrict__ vals,
                                                         int32_t* __restrict__ seg) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const int64_t key = (int64_t)tok[i] - v0;
    keys[i] = (key >= 0 && key < vr) ? (uint32_t)key : (uint32_t)vr;
    vals[i] = (uint32_t)i;
  }
  if (i < vr) seg[i] = -1;
}

// Stable LSD radix sort of (key, val) pairs by key, 8-bit digits, one
// workgroup of 1024 threads. Each pass: digit histogram (LDS integer atomics),
// exclusive scan, then tiles of 1024 elements in order: an element's rank
// among equal digits before it in the tile comes from 8 wave ballots (lanes
// with the same digit) and the per-wave digit counts of the lower waves.
// Ping-pongs between (k0, v0) and (k1, v1); the result ends in (k0, v0) when
// `passes` is even, else in (k1, v1).
constexpr int kSortThreads = 1024, kSortWaves = kSortThreads / 64;
__global__ __launch_bounds__(kSortThreads) void radix_sort_kernel(uint32_t* k0, uint32_t* v0_, uint32_t* k1,
                                                                  uint32_t* v1, int n, int passes) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int wcnt[kSortWaves][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
  uint32_t *ki = k0, *vi = v0_, *ko = k1, *vo = v1;
  for (int p = 0; p < passes; ++p) {
    const int shift = 8 * p;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSortThreads) atomicAdd(&hist[(ki[i] >> shift) & 255], 1);
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int d = 0; d < 256; ++d) {
        base[d] = run;
        run += hist[d];
      }
    }
    __syncthreads();
    for (int t0 = 0; t0 < n; t0 += kSortThreads) {
      for (int d = tid; d < kSortWaves * 256; d += kSortThreads) (&wcnt[0][0])[d] = 0;
      __syncthreads();
      const int i = t0 + tid;
      const bool live = i < n;
      const uint32_t key = live ? ki[i] : 0u, val = live ? vi[i] : 0u;
      const int d = (int)((key >> shift) & 255);
      uint64_t same = __ballot(live);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t bit = __ballot(live && ((d >> b) & 1));
        same &= ((d >> b) & 1) ? bit : ~bit;
      }
      const int rank = __popcll(same & lt);
      if (live && rank == 0) wcnt[wave][d] = __popcll(same);
      __syncthreads();
      if (live) {
        int off = base[d] + rank;
        for (int w = 0; w < wave; ++w) off += wcnt[w][d];
        ko[off] = key;
        vo[off] = val;
      }
      __syncthreads();
      if (tid < 256) {
        int add = 0;
        for (int w = 0; w < kSortWaves; ++w) add += wcnt[w][tid];
        base[tid] += add;
      }
      __syncthreads();
    }
    uint32_t* t;
    t = ki; ki = ko; ko = t;
    t = vi; vi = vo; vo = t;
  }
}

// seg[v] = first position of key v in the sorted keys.
__global__ __launch_bounds__(256) void embed_segments_kernel(const uint32_t* __restrict__ keys, int n, int vr,
                                                             int32_t* __restrict__ seg) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t k = keys[i];
  if (k < (uint32_t)vr && (i == 0 || keys[i - 1] != k)) seg[k] = i;
}

// d_emb[v][chunk] = sum over the sorted rows of key v, ascending row order,
// of d_out[row][chunk] (zeros for rows no id points to).
template <typename T>
__global__ __launch_bounds__(256) void embed_grad_kernel(const T* __restrict__ d_out, const uint32_t* __restrict__ keys,
                                                         const uint32_t* __restrict__ vals,
                                                         const int32_t* __restrict__ seg, int n, int vr, int cpr,
                                                         float* __restrict__ d_emb) {
  constexpr int V = Vec16<T>::N;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)vr * cpr) return;
  const int v = (int)(c / cpr), j = (int)(c % cpr);
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  const int s = seg[v];
  if (s >= 0) {
    for (int i = s; i < n && keys[i] == (uint32_t)v; ++i) {
      Vec16<T> x;
      x.raw = ld16(d_out + (int64_t)vals[i] * cpr * V + j * V);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += to_f32(x.get(e));
    }
  }
  float* o = d_emb + c * V;
#pragma unroll
  for (int e = 0; e < V; e += 4) *reinterpret_cast<f32x4*>(o + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
}

int sort_passes(int vr) {
  int bits = 0;
  while ((1ll << bits) <= vr) ++bits;   // keys go up to vr (the out-of-range marker)
  return (bits + 7) / 8;
}

}  // namespace

size_t embedding_ws_bytes(int64_t rows, int vr) { return ((size_t)rows * 4 + (size_t)vr + 64) * 4; }

hipError_t launch_embedding_fwd(int dtype, const int32_t* tokens, const void* emb, void* out, int64_t rows, int cols,
                                int64_t v0, int vr, hipStream_t s) {
  TraceScope trace(K_EMB_FWD, s, (double)rows * cols * 2 * dtype_size(dtype) + rows * 4.0);
  if (rows == 0) return hipSuccess;
  const int v = dtype == DT_BF16 ? 8 : 4;
  const int cpr = cols / v;
  const int64_t nchunks = rows * cpr;
  if (nchunks >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((nchunks + 255) / 256));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(embed_fwd_kernel<bf16>, grid, dim3(256), 0, s, tokens, static_cast<const bf16*>(emb),
                       static_cast<bf16*>(out), v0, vr, cpr, (uint32_t)nchunks);
  else
    hipLaunchKernelGGL(embed_fwd_kernel<float>, grid, dim3(256), 0, s, tokens, static_cast<const float*>(emb),
                       static_cast<float*>(out), v0, vr, cpr, (uint32_t)nchunks);
  return hipGetLastError();
}

hipError_t launch_embedding_bwd(int dtype, const int32_t* tokens, const void* d_out, float* d_emb, int64_t rows,
                                int cols, int64_t v0, int vr, void* ws, hipStream_t s) {
  if (rows >= (int64_t(1) << 31) || vr <= 0) return hipErrorInvalidValue;
  const int n = (int)rows;
  uint32_t* k0 = static_cast<uint32_t*>(ws);
  uint32_t* va = k0 + rows;
  uint32_t* k1 = va + rows;
  uint32_t* vb = k1 + rows;
  int32_t* seg = reinterpret_cast<int32_t*>(vb + rows);
  const int passes = sort_passes(vr);
  uint32_t* keys = (passes & 1) ? k1 : k0;
  uint32_t* vals = (passes & 1) ? vb : va;
  hipError_t e;
  {
    TraceScope trace(K_EMB_SORT, s, (double)rows * 16.0 * passes);
    const int64_t m = std::max<int64_t>(rows, vr);
    hipLaunchKernelGGL(embed_keys_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, tokens, n, v0, vr, k0,
                       va, seg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (n > 0) {
      hipLaunchKernelGGL(radix_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, k0, va, k1, vb, n, passes);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(embed_segments_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, keys, n, vr,
                         seg);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  TraceScope trace(K_EMB_BWD, s, (double)rows * cols * dtype_size(dtype) + (double)vr * cols * 4);
  const int v = dtype == DT_BF16 ? 8 : 4;
  const int cpr = cols / v;
  const int64_t total = (int64_t)vr * cpr;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(embed_grad_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(d_out), keys, vals,
                       seg, n, vr, cpr, d_emb);
  else
    hipLaunchKernelGGL(embed_grad_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(d_out), keys,
                       vals, seg, n, vr, cpr, d_emb);
  return hipGetLastError();
}


// ------------------------------------------------------------------ loss rows
// Gather of the rows a masked loss is taken on, and the expansion of their
// gradient back to every row (zeros elsewhere). One thread per W-byte unit
// (W = 16 when the rows and pointers allow, else 4); every index is checked
// against the source's row count, so a bad index reads nothing.
namespace {
template <int W>
struct Unit;
template <>
struct Unit<16> { using T = u32x4; };
template <>
struct Unit<4> { using T = uint32_t; };

template <int W>
__global__ __launch_bounds__(256) void rows_gather_kernel(const char* __restrict__ src, const int32_t* __restrict__ rows,
                                                          int64_t n, int64_t n_src, int64_t row_bytes,
                                                          char* __restrict__ dst) {
  using U = typename Unit<W>::T;
  const int64_t upr = row_bytes / W;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n * upr) return;
  const int64_t i = u / upr, c = u % upr;
  const int64_t r = rows[i];
  U v{};
  if (r >= 0 && r < n_src) v = *reinterpret_cast<const U*>(src + r * row_bytes + c * W);
  *reinterpret_cast<U*>(dst + i * row_bytes + c * W) = v;
}

template <int W>
__global__ __launch_bounds__(256) void rows_expand_kernel(const char* __restrict__ src, const int32_t* __restrict__ pos,
                                                          int64_t n_dst, int64_t n_src, int64_t row_bytes,
                                                          char* __restrict__ dst) {
  using U = typename Unit<W>::T;
  const int64_t upr = row_bytes / W;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n_dst * upr) return;
  const int64_t r = u / upr, c = u % upr;
  const int64_t p = pos[r];
  U v{};
  if (p >= 0 && p < n_src) v = *reinterpret_cast<const U*>(src + p * row_bytes + c * W);
  *reinterpret_cast<U*>(dst + r * row_bytes + c * W) = v;
}

bool wide_units(const void* a, const void* b, int64_t row_bytes) {
  return row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(a) % 16 == 0 && reinterpret_cast<uintptr_t>(b) % 16 == 0;
}
}  // namespace

hipError_t launch_rows_gather(const void* src, const int32_t* rows, int64_t n, int64_t n_src, int64_t row_bytes,
                              void* dst, hipStream_t s) {
  TraceScope trace(K_ROWS_GATHER, s, 2.0 * (double)n * row_bytes + 4.0 * n);
  if (n == 0) return hipSuccess;
  const bool w16 = wide_units(src, dst, row_bytes);
  const int64_t units = n * (row_bytes / (w16 ? 16 : 4));
  const dim3 grid((unsigned)((units + 255) / 256));
  if (w16)
    hipLaunchKernelGGL(rows_gather_kernel<16>, grid, dim3(256), 0, s, static_cast<const char*>(src), rows, n, n_src,
                       row_bytes, static_cast<char*>(dst));
  else
    hipLaunchKernelGGL(rows_gather_kernel<4>, grid, dim3(256), 0, s, static_cast<const char*>(src), rows, n, n_src,
                       row_bytes, static_cast<char*>(dst));
  return hipGetLastError();
}

hipError_t launch_rows_expand(const void* src, const int32_t* pos, int64_t n_dst, int64_t n_src, int64_t row_bytes,
                              void* dst, hipStream_t s) {
  TraceScope trace(K_ROWS_EXPAND, s, (double)n_dst * row_bytes + (double)n_src * row_bytes + 4.0 * n_dst);
  if (n_dst == 0) return hipSuccess;
  const bool w16 = wide_units(src, dst, row_bytes);
  const int64_t units = n_dst * (row_bytes / (w16 ? 16 : 4));
  const dim3 grid((unsigned)((units + 255) / 256));
  if (w16)
    hipLaunchKernelGGL(rows_expand_kernel<16>, grid, dim3(256), 0, s, static_cast<const char*>(src), pos, n_dst, n_src,
                       row_bytes, static_cast<char*>(dst));
  else
    hipLaunchKernelGGL(rows_expand_kernel<4>, grid, dim3(256), 0, s, static_cast<const char*>(src), pos, n_dst, n_src,
                       row_bytes, static_cast<char*>(dst));
  return hipGetLastError();
}

}  // namespace tpl
