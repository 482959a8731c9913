// Vocabulary-parallel cross-entropy (guide page section 3.3; podcast page
// Outline: the output embedding is split along the vocabulary and the gather
// is deferred into the loss). Each rank reduces its logits shard to three
// numbers per row -- running max m, sum of exp(l - m), target logit (or 0) --
// so the softmax over the shard is never written; ranks then exchange only
// these [N, 3] statistics, combined by log-sum-exp rescaling.
#include "common.h"
#include "kernels.h"

namespace tpl {
namespace {

// Merge (m, s) pairs of the online log-sum-exp.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

// One workgroup per row: stats[row] = (max, sum exp(l - max), target logit or 0).
// Each thread takes chunks of 16 B in groups of kU (loads of a group issued
// together, then merged into the running (max, sum)), so enough bytes are in
// flight to stream the logits at HBM rate.
template <typename T>
__global__ __launch_bounds__(256) void xent_stats_kernel(const T* __restrict__ logits, int vr,
                                                         const int32_t* __restrict__ targets, int64_t v0,
                                                         float* __restrict__ stats) {
  constexpr int V = Vec16<T>::N, kU = 4;
  const int64_t row = blockIdx.x;
  const T* lr = logits + row * vr;
  const int nch = vr / V;
  float m = -INFINITY, s = 0.f;
  for (int base = threadIdx.x; base < nch; base += 256 * kU) {
    Vec16<T> x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int ch = base + 256 * u;
      if (ch < nch) x[u].raw = ld16(lr + ch * V);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (base + 256 * u < nch)
#pragma unroll
        for (int e = 0; e < V; ++e) mx = fmaxf(mx, to_f32(x[u].get(e)));
    const float mn = fmaxf(m, mx);
    float acc = s * __expf(m - mn);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (base + 256 * u < nch)
#pragma unroll
        for (int e = 0; e < V; ++e) acc += __expf(to_f32(x[u].get(e)) - mn);
    m = mn;
    s = acc;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
    lse_merge(m, s, m2, s2);
  }
  __shared__ float sm[4], ss[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[wave] = m; ss[wave] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int w = 1; w < 4; ++w) lse_merge(M, S, sm[w], ss[w]);
    const int64_t t = (int64_t)targets[row] - v0;
    const float tl = (t >= 0 && t < vr) ? to_f32(lr[t]) : 0.f;
    stats[row * 3 + 0] = M;
    stats[row * 3 + 1] = S;
    stats[row * 3 + 2] = tl;
  }
}

// stats[row] from the per-tile (max, sum exp) pairs of the fused logits
// product: 64 rows per workgroup (lane = row), wave w of 16 merges the w-th
// slice of the tile columns in order, then the slices are merged in order --
// a fixed order, so the result is deterministic. The target logit is read
// from the stored logits.
template <typename T>
__global__ __launch_bounds__(1024) void xent_merge_kernel(const float* __restrict__ xpart, int tcols, int64_t rows,
                                                          const T* __restrict__ logits, int vr,
                                                          const int32_t* __restrict__ targets, int64_t v0,
                                                          float* __restrict__ stats) {
  __shared__ float q[16][64][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 64 + lane;
  const int per = (tcols + 15) / 16;
  const int t0 = wave * per, t1 = min(tcols, t0 + per);
  float m = -INFINITY, s = 0.f;
  if (row < rows) {
    constexpr int kB = 8;   // loads of a batch in flight together, then merged in order
    for (int t = t0; t < t1; t += kB) {
      float2 p[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (t + u < t1) p[u] = *reinterpret_cast<const float2*>(xpart + ((int64_t)(t + u) * rows + row) * 2);
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (t + u < t1) lse_merge(m, s, p[u].x, p[u].y);
    }
  }
  q[wave][lane][0] = m;
  q[wave][lane][1] = s;
  __syncthreads();
  if (wave == 0 && row < rows) {
    float M = q[0][lane][0], S = q[0][lane][1];
    for (int w = 1; w < 16; ++w) lse_merge(M, S, q[w][lane][0], q[w][lane][1]);
    const int64_t t = (int64_t)targets[row] - v0;
    stats[row * 3 + 0] = M;
    stats[row * 3 + 1] = S;
    stats[row * 3 + 2] = (t >= 0 && t < vr) ? to_f32(logits[row * vr + t]) : 0.f;
  }
}

struct StatPtrs { const float* p[64]; };

// Single workgroup: combine the t ranks' statistics, per-row loss and the
// masked mean (fixed reduction order -> deterministic).
__global__ __launch_bounds__(1024) void xent_finish_kernel(StatPtrs st, int t, int64_t rows,
                                                           const uint8_t* __restrict__ mask,
                                                           float* __restrict__ lse, float* __restrict__ loss_rows,
                                                           float* __restrict__ loss) {
  float acc = 0.f, cnt = 0.f;
  constexpr int kB = 8;   // rows per thread whose loads are in flight together
  for (int64_t r0 = threadIdx.x; r0 < rows; r0 += 1024 * kB) {
    float M[kB], S[kB], TL[kB], w[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) { M[u] = -INFINITY; S[u] = 0.f; TL[u] = 0.f; w[u] = 0.f; }
    for (int k = 0; k < t; ++k) {
      float mk[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int64_t r = r0 + 1024 * u;
        mk[u] = r < rows ? st.p[k][r * 3] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) M[u] = fmaxf(M[u], mk[u]);
    }
    for (int k = 0; k < t; ++k) {
      float mk[kB], sk[kB], tk[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int64_t r = r0 + 1024 * u;
        mk[u] = 0.f; sk[u] = 0.f; tk[u] = 0.f;
        if (r < rows) { mk[u] = st.p[k][r * 3]; sk[u] = st.p[k][r * 3 + 1]; tk[u] = st.p[k][r * 3 + 2]; }
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        S[u] += sk[u] * __expf(mk[u] - M[u]);
        TL[u] += tk[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int64_t r = r0 + 1024 * u;
      if (r < rows) w[u] = mask ? (float)mask[r] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int64_t r = r0 + 1024 * u;
      if (r < rows) {
        const float l = M[u] + __logf(S[u]);
        const float lr = w[u] * (l - TL[u]);
        lse[r] = l;
        loss_rows[r] = lr;
        acc += lr;
        cnt += w[u];
      }
    }
  }
  __shared__ float sa[16], sc[16];
  acc = wave_sum(acc);
  cnt = wave_sum(cnt);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sa[wave] = acc; sc[wave] = cnt; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float A = 0.f, C = 0.f;
    for (int w = 0; w < 16; ++w) { A += sa[w]; C += sc[w]; }
    loss[0] = C > 0.f ? A / C : 0.f;
    loss[1] = C;
  }
}

// The same for t <= 8 ranks: each thread loads all ranks' (max, sum, target
// logit) of its kB rows at once, so one round of load latency serves a batch
// instead of 2t dependent rounds. Ranks past t read as (-inf, 0, 0): the max
// is unchanged and the sums gain exact zeros after rank t-1, so the results
// equal xent_finish_kernel's bit for bit.
__global__ __launch_bounds__(1024) void xent_finish8_kernel(StatPtrs st, int t, int64_t rows,
                                                            const uint8_t* __restrict__ mask,
                                                            float* __restrict__ lse, float* __restrict__ loss_rows,
                                                            float* __restrict__ loss) {
  constexpr int kB = 2;
  float acc = 0.f, cnt = 0.f;
  for (int64_t r0 = threadIdx.x; r0 < rows; r0 += 1024 * kB) {
    float mk[8][kB], sk[8][kB], tk[8][kB];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int64_t r = r0 + 1024 * u;
        mk[k][u] = -INFINITY; sk[k][u] = 0.f; tk[k][u] = 0.f;
        if (k < t && r < rows) {
          mk[k][u] = st.p[k][r * 3];
          sk[k][u] = st.p[k][r * 3 + 1];
          tk[k][u] = st.p[k][r * 3 + 2];
        }
      }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int64_t r = r0 + 1024 * u;
      if (r >= rows) continue;
      float M = -INFINITY, S = 0.f, TL = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) M = fmaxf(M, mk[k][u]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k < t) {
          S += sk[k][u] * __expf(mk[k][u] - M);
          TL += tk[k][u];
        }
      }
      const float w = mask ? (float)mask[r] : 1.f;
      const float l = M + __logf(S);
      const float lr = w * (l - TL);
      lse[r] = l;
      loss_rows[r] = lr;
      acc += lr;
      cnt += w;
    }
  }
  __shared__ float sa[16], sc[16];
  acc = wave_sum(acc);
  cnt = wave_sum(cnt);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sa[wave] = acc; sc[wave] = cnt; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float A = 0.f, C = 0.f;
    for (int w = 0; w < 16; ++w) { A += sa[w]; C += sc[w]; }
    loss[0] = C > 0.f ? A / C : 0.f;
    loss[1] = C;
  }
}

// In place: l <- g (exp(l - lse) - [j == target - v0]), g = dloss * mask / count.
// Streams the [rows][vr] logits as one flat array of 16-B chunks (kU chunks
// per thread, loads issued together); the per-row scalars are re-read per
// chunk from cache. Loads and stores carry the non-temporal hint: the array
// is far larger than the caches, and with ordinary stores the products that
// read dlogits next ran ~2% slower (gemm_nn on the gpt2 shard 1020 -> 997 us),
// while this kernel's own time did not change.
template <typename T>
__global__ __launch_bounds__(256) void xent_dlogits_kernel(T* logits, int vr, int64_t nchunks,
                                                           const int32_t* __restrict__ targets, int64_t v0,
                                                           const uint8_t* __restrict__ mask,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ loss, float dloss) {
  constexpr int V = Vec16<T>::N, kU = 4;
  const int cpr = vr / V;   // chunks per row
  const float cnt = loss[1];
  const float gs = cnt > 0.f ? dloss / cnt : 0.f;
  const int64_t base = ((int64_t)blockIdx.x * kU) * 256 + threadIdx.x;
  Vec16<T> x[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t c = base + 256 * u;
    if (c < nchunks) x[u].raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(logits + c * V));
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t c = base + 256 * u;
    if (c < nchunks) {
      const uint32_t row = (uint32_t)c / (uint32_t)cpr;   // nchunks < 2^32 (checked by the launcher)
      const int j0 = (int)((uint32_t)c - row * (uint32_t)cpr) * V;
      const float g = (mask ? (float)mask[row] : 1.f) * gs;
      const float L = lse[row];
      const int64_t t = (int64_t)targets[row] - v0 - j0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float p = __expf(to_f32(x[u].get(e)) - L);
        if (e == t) p -= 1.f;
        x[u].set(e, from_f32<T>(g * p));
      }
      __builtin_nontemporal_store(x[u].raw, reinterpret_cast<u32x4*>(logits + c * V));
    }
  }
}

}  // namespace

hipError_t launch_xent_stats(int dtype, const void* logits, int64_t rows, int vr, const int32_t* targets,
                             int64_t v0, float* stats, hipStream_t s) {
  TraceScope trace(K_XENT_STATS, s, (double)rows * vr * dtype_size(dtype) + rows * 16.0);
  if (rows == 0) return hipSuccess;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(xent_stats_kernel<bf16>, dim3((unsigned)rows), dim3(256), 0, s,
                       static_cast<const bf16*>(logits), vr, targets, v0, stats);
  else
    hipLaunchKernelGGL(xent_stats_kernel<float>, dim3((unsigned)rows), dim3(256), 0, s,
                       static_cast<const float*>(logits), vr, targets, v0, stats);
  return hipGetLastError();
}

hipError_t launch_xent_merge(int dtype, const float* xpart, int tcols, int64_t rows, const void* logits, int vr,
                             const int32_t* targets, int64_t v0, float* stats, hipStream_t s) {
  TraceScope trace(K_XENT_MERGE, s, (double)rows * (8.0 * tcols + 12 + 6));
  if (rows == 0) return hipSuccess;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(xent_merge_kernel<bf16>, dim3((unsigned)((rows + 63) / 64)), dim3(1024), 0, s, xpart, tcols, rows,
                       static_cast<const bf16*>(logits), vr, targets, v0, stats);
  else
    hipLaunchKernelGGL(xent_merge_kernel<float>, dim3((unsigned)((rows + 63) / 64)), dim3(1024), 0, s, xpart, tcols,
                       rows, static_cast<const float*>(logits), vr, targets, v0, stats);
  return hipGetLastError();
}

hipError_t launch_xent_finish(const float* const* all_stats, int t, int64_t rows, const uint8_t* mask, float* lse,
                              float* loss_rows, float* loss, hipStream_t s) {
  TraceScope trace(K_XENT_FINISH, s, (double)rows * (12.0 * t + 9));
  StatPtrs sp;
  for (int i = 0; i < 64; ++i) sp.p[i] = i < t ? all_stats[i] : nullptr;
  if (t <= 8)
    hipLaunchKernelGGL(xent_finish8_kernel, dim3(1), dim3(1024), 0, s, sp, t, rows, mask, lse, loss_rows, loss);
  else
    hipLaunchKernelGGL(xent_finish_kernel, dim3(1), dim3(1024), 0, s, sp, t, rows, mask, lse, loss_rows, loss);
  return hipGetLastError();
}

hipError_t launch_xent_dlogits(int dtype, void* logits, int64_t rows, int vr, const int32_t* targets, int64_t v0,
                               const uint8_t* mask, const float* lse, const float* loss, float dloss, hipStream_t s) {
  TraceScope trace(K_XENT_DLOGITS, s, (double)rows * vr * 2 * dtype_size(dtype) + rows * 9.0);
  if (rows == 0) return hipSuccess;
  const int v = dtype == DT_BF16 ? 8 : 4;
  const int64_t nchunks = rows * (vr / v);
  if (nchunks >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((nchunks + 1023) / 1024));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(xent_dlogits_kernel<bf16>, grid, dim3(256), 0, s, static_cast<bf16*>(logits), vr, nchunks,
                       targets, v0, mask, lse, loss, dloss);
  else
    hipLaunchKernelGGL(xent_dlogits_kernel<float>, grid, dim3(256), 0, s, static_cast<float*>(logits), vr, nchunks,
                       targets, v0, mask, lse, loss, dloss);
  return hipGetLastError();
}

}  // namespace tpl
