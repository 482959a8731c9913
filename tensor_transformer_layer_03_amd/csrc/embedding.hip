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
#include <mutex>

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

// In-LDS sort for up to kLdsSortMax rows, one workgroup of 1024 threads, in
// one launch that also derives the keys from the ids and writes seg[]. Each
// row becomes one 32-bit word (key << ib) | row, ib = bits of the largest row
// index; the words are all distinct, so ordering them by key alone, stably,
// is the same as ordering (key, row) pairs. LSD radix passes over the key in
// 4-bit digits; between passes thread t holds rows [E*t, E*t + E) in order
// (E = ceil(n / 1024) <= 8) in registers. In a pass each thread counts its
// digits in a 64-bit word of 4-bit counters (an element's rank among its
// thread's equal digits is the counter before the increment), the 16 x 1024
// counts, digit-major then thread, are scanned across the workgroup, and
// every element goes to base[digit][thread] + rank in LDS: stable, since the
// scan order is the element order within each digit. Global loads and stores
// run in the coalesced order j = tid + 1024 q through LDS. seg[] is written
// at the first occurrence of each key present only; the gradient kernel
// accepts an entry only where it points at that first occurrence, so the
// other entries are never cleared.
constexpr int kLdsSortMax = 8192, kLdsSortE = kLdsSortMax / kSortThreads;
__global__ __launch_bounds__(kSortThreads) void embed_sort_lds_kernel(const int32_t* __restrict__ tok, int n,
                                                                      int64_t v0, int vr, int ib, int passes,
                                                                      uint32_t* __restrict__ keys,
                                                                      uint32_t* __restrict__ vals,
                                                                      int32_t* __restrict__ seg) {
  __shared__ uint32_t buf[kLdsSortMax];
  __shared__ __attribute__((aligned(16))) uint32_t cnt[16 * kSortThreads];   // [digit][thread]
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kSortWaves];
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t t8[kLdsSortE];
#pragma unroll
  for (int q = 0; q < kLdsSortE; ++q) t8[q] = tok[min(tid + q * kSortThreads, n - 1)];
#pragma unroll
  for (int q = 0; q < kLdsSortE; ++q) {
    const int j = tid + q * kSortThreads;
    const int64_t key = (int64_t)t8[q] - v0;
    const uint32_t k = (key >= 0 && key < vr) ? (uint32_t)key : (uint32_t)vr;
    if (j < n) buf[j] = (k << ib) | (uint32_t)j;
  }
  __syncthreads();
  const int E = (n + kSortThreads - 1) / kSortThreads;
  const int first = tid * E;
  const int own = max(0, min(E, n - first));   // rows this thread holds
  uint32_t w[kLdsSortE];
#pragma unroll
  for (int e = 0; e < kLdsSortE; ++e) w[e] = buf[min(first + e, n - 1)];
  for (int p = 0; p < passes; ++p) {
    const int shift = ib + 4 * p;
    uint64_t c = 0;
    uint32_t rk[kLdsSortE];
#pragma unroll
    for (int e = 0; e < kLdsSortE; ++e) {
      const int d4 = (int)((w[e] >> shift) & 15u) * 4;
      rk[e] = (uint32_t)(c >> d4) & 15u;
      if (e < own) c += 1ull << d4;
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d * kSortThreads + tid] = (uint32_t)(c >> (4 * d)) & 15u;
    __syncthreads();
    // exclusive scan of cnt in index order: thread t takes entries [16t, 16t + 16)
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 x = *reinterpret_cast<const uint4*>(&cnt[16 * tid + 4 * q]);
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t x = v[j];
      v[j] = tot;
      tot += x;
    }
    uint32_t inc = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t base = inc - tot;
#pragma unroll
    for (int q = 0; q < kSortWaves; q += 4) {   // + the totals of the lower waves
      const uint4 x = *reinterpret_cast<const uint4*>(&wsum[q]);
      base += (q < wave ? x.x : 0u) + (q + 1 < wave ? x.y : 0u) + (q + 2 < wave ? x.z : 0u) + (q + 3 < wave ? x.w : 0u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(&cnt[16 * tid + 4 * q]) =
          uint4{base + v[4 * q], base + v[4 * q + 1], base + v[4 * q + 2], base + v[4 * q + 3]};
    __syncthreads();
    uint32_t pos[kLdsSortE];
#pragma unroll
    for (int e = 0; e < kLdsSortE; ++e) pos[e] = cnt[(int)((w[e] >> shift) & 15u) * kSortThreads + tid] + rk[e];
#pragma unroll
    for (int e = 0; e < kLdsSortE; ++e)
      if (e < own) buf[pos[e]] = w[e];
    __syncthreads();
    if (p + 1 < passes) {
#pragma unroll
      for (int e = 0; e < kLdsSortE; ++e) w[e] = buf[min(first + e, n - 1)];
    }
  }
  const uint32_t imask = (1u << ib) - 1u;
#pragma unroll
  for (int q = 0; q < kLdsSortE; ++q) {
    const int j = tid + q * kSortThreads;
    if (j < n) {
      const uint32_t x = buf[j], k = x >> ib;
      keys[j] = k;
      vals[j] = x & imask;
      if (k < (uint32_t)vr && (j == 0 || (buf[j - 1] >> ib) != k)) seg[k] = j;
    }
  }
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
  // seg[v] counts only where it is the first position of key v (stale entries fail the test)
  const int s = seg[v];
  if (s >= 0 && s < n && keys[s] == (uint32_t)v && (s == 0 || keys[s - 1] != (uint32_t)v)) {
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

int key_bits(int vr) {
  int bits = 0;
  while ((1ll << bits) <= vr) ++bits;   // keys go up to vr (the out-of-range marker)
  return bits;
}

int index_bits(int n) {
  int bits = 0;
  while ((1ll << bits) < n) ++bits;
  return bits;
}

}  // namespace

size_t embedding_ws_bytes(int64_t rows, int vr) { return ((size_t)rows * 4 + (size_t)vr + 64) * 4; }

// ------------------------------------------------------------------ allocation-free backward
// The workspace of the allocation-free backward lives in this file-scope
// device array, one copy per GPU, held until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept per device. Nothing in it must start at zero: the sort writes every
// key and value it reads back, and the gradient kernel accepts a segment
// start only where it points at the first occurrence of its key (the
// multi-pass sort clears the segment table itself).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

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
  const int kb = key_bits(vr), ib = index_bits(n);
  const bool in_lds = n <= kLdsSortMax && ib + kb <= 32;
  const int passes = (kb + 7) / 8;
  uint32_t* keys = (!in_lds && (passes & 1)) ? k1 : k0;
  uint32_t* vals = (!in_lds && (passes & 1)) ? vb : va;
  hipError_t e;
  if (in_lds) {
    TraceScope trace(K_EMB_SORT, s, (double)rows * 12.0 + (double)vr * 4.0);
    hipLaunchKernelGGL(embed_sort_lds_kernel, dim3(1), dim3(kSortThreads), 0, s, tokens, n, v0, vr, ib, (kb + 3) / 4,
                       keys, vals, seg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
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
