// Memory-bound kernels of the two variants the pages measure the fused loss
// against (aib.vote summary, paragraph comparing Dense KL, Forward-chunked KL
// and Fused chunked KL; Hugging Face blog "Making Knowledge Distillation
// Cheap Enough to Run at Scale", sections "Two systems changes" and "Scaling
// to long context lengths"):
//   dense KL:           the student's full log-probability grid and the
//                       teacher's full probability grid rebuilt from the
//                       cached top-K, compared element by element;
//   forward-chunked KL: the student's full logit grid, computed and kept for
//                       the backward pass, with a sparse teacher.
// Row statistics of stored logits, in-place log-softmax, the dense teacher
// grid, the dense KL, the gather from stored logits and the logit gradient
// formed from stored grids.  One 256-thread workgroup per row; every
// reduction runs in a fixed order.  Grid rows have a pitch of ldz floats (a
// multiple of 4, so every row starts 16-byte aligned).
#include <hip/hip_runtime.h>

#include "kd_internal.h"

namespace kd {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kT = 256;  // threads per row

__device__ inline float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Online (max, sum of exp(x - max)) of one more element.
__device__ inline void lse_push(float& m, float& s, float x) {
  if (x == kNegInf) return;
  if (x > m) {
    s = s * exp_fast(m - x) + 1.f;
    m = x;
  } else {
    s += exp_fast(x - m);
  }
}

__device__ inline float2 lse_merge(float2 a, float2 b) {
  const float m = fmaxf(a.x, b.x);
  if (m == kNegInf) return make_float2(kNegInf, 0.f);
  return make_float2(m, a.y * exp_fast(a.x - m) + b.y * exp_fast(b.x - m));
}

// (max, sum-exp) of the whole workgroup: a butterfly within each wavefront
// (every lane ends with the same value: the merge is commutative), then the
// four wavefronts in order.
__device__ inline float2 block_lse(float2 a, float2* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = lse_merge(a, make_float2(__shfl_xor(a.x, o, 64), __shfl_xor(a.y, o, 64)));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
  __syncthreads();
  float2 r = lse_merge(lse_merge(lse_merge(sh[0], sh[1]), sh[2]), sh[3]);
  __syncthreads();
  return r;
}

__device__ inline float block_sum(float a, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
  __syncthreads();
  const float r = ((sh[0] + sh[1]) + sh[2]) + sh[3];
  __syncthreads();
  return r;
}

// (max, sum-exp) of z[0..V), 16-byte loads where the row allows.
__device__ inline float2 row_stats(const float* z, int V, float2* sh) {
  float m = kNegInf, s = 0.f;
  const int V4 = V >> 2;
  for (int q = threadIdx.x; q < V4; q += kT) {
    const float4 x = reinterpret_cast<const float4*>(z)[q];
    lse_push(m, s, x.x);
    lse_push(m, s, x.y);
    lse_push(m, s, x.z);
    lse_push(m, s, x.w);
  }
  for (int v = 4 * V4 + threadIdx.x; v < V; v += kT) lse_push(m, s, z[v]);
  return block_lse(make_float2(m, s), sh);
}

// part[r] = (max, sum-exp) of logit row r (one vocabulary "tile" per row).
__global__ __launch_bounds__(kT) void row_stats_kernel(const float* __restrict__ Z, long long ldz, int V,
                                                       float2* __restrict__ part) {
  __shared__ float2 sh[4];
  const float2 t = row_stats(Z + (long long)blockIdx.x * ldz, V, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = t;
}

// Row r of the grid becomes log q = z - LSE(z) in place; lse[c0 + r] = LSE.
__global__ __launch_bounds__(kT) void log_softmax_kernel(float* __restrict__ Z, long long ldz, int V, int c0,
                                                         float* __restrict__ lse) {
  __shared__ float2 sh[4];
  float* z = Z + (long long)blockIdx.x * ldz;
  const float2 t = row_stats(z, V, sh);
  const float L = t.x + __logf(t.y);
  if (threadIdx.x == 0) lse[c0 + blockIdx.x] = L;
  for (int v = threadIdx.x; v < V; v += kT) z[v] -= L;
}

// Row r of the dense teacher grid: p of the row's cached entries at their
// ids, 0 elsewhere (and everywhere on a masked row).  p holds, for an id a
// row repeats, the sum of its occurrences' p at the first one and 0 at the
// others, so a repeated id is written once, with the sum.
__global__ __launch_bounds__(kT) void teacher_grid_kernel(float* __restrict__ P, long long ldz, int V, int c0,
                                                          const int* __restrict__ idx, const float* __restrict__ p,
                                                          const uint8_t* __restrict__ mask, int K) {
  float* row = P + (long long)blockIdx.x * ldz;
  for (int v = threadIdx.x; v < V; v += kT) row[v] = 0.f;
  __syncthreads();
  const int t = c0 + blockIdx.x;
  if (mask != nullptr && mask[t] == 0) return;
  for (int k = threadIdx.x; k < K; k += kT) {
    const int v = idx[(long long)t * K + k];
    const float pk = p[(long long)t * K + k];
    if (v >= 0 && v < V && pk > 0.f) row[v] = pk;
  }
}

// row_kl[c0 + r] = sum_v P (log P - log q) over the whole vocabulary
// (0 log 0 := 0), 0 on masked rows.
__global__ __launch_bounds__(kT) void dense_kl_kernel(const float* __restrict__ P, const float* __restrict__ LQ,
                                                      long long ldz, int V, int c0,
                                                      const uint8_t* __restrict__ mask, float* __restrict__ row_kl) {
  __shared__ float sh[4];
  const int t = c0 + blockIdx.x;
  const float* pr = P + (long long)blockIdx.x * ldz;
  const float* lq = LQ + (long long)blockIdx.x * ldz;
  float a = 0.f;
  for (int v = threadIdx.x; v < V; v += kT) {
    const float pv = pr[v];
    if (pv > 0.f) a += pv * (__logf(pv) - lq[v]);
  }
  a = block_sum(a, sh);
  if (threadIdx.x == 0) row_kl[t] = (mask != nullptr && mask[t] == 0) ? 0.f : a;
}

// g[t][k] = Z[r][i_{t,k}] of the stored logits, t = c0 + r (unmasked rows,
// valid ids).
__global__ __launch_bounds__(kT) void gather_kernel(const float* __restrict__ Z, long long ldz, int rows, int c0,
                                                    const int* __restrict__ idx, const uint8_t* __restrict__ mask,
                                                    int K, int V, float* __restrict__ g) {
  const long long e = (long long)blockIdx.x * kT + threadIdx.x;
  if (e >= (long long)rows * K) return;
  const int r = (int)(e / K), k = (int)(e - (long long)r * K);
  const int t = c0 + r;
  if (mask != nullptr && mask[t] == 0) return;
  const int v = idx[(long long)t * K + k];
  if (v >= 0 && v < V) g[(long long)t * K + k] = Z[(long long)r * ldz + v];
}

// Row r (< c_pad) of the chunk's logit gradient, rounded to bf16, in G (row
// pitch v_pad, zero at v >= V and on rows r >= rows):
//   dense:           G = gw (S_t exp(log q) - P)           from the two grids
//   forward-chunked: G = gw (S_t exp(z - LSE_t)) - gw p_k at (t, i_{t,k})
// with gw = grad_loss * [mask_t] / N_valid, the fused path's G.
template <bool kDense>
__global__ __launch_bounds__(kT) void grad_kernel(const float* __restrict__ Z, const float* __restrict__ P,
                                                  long long ldz, int V, int v_pad, int rows, int c0,
                                                  const float* __restrict__ lse, const float* __restrict__ S,
                                                  const uint8_t* __restrict__ mask, const Ctrl* __restrict__ ctrl,
                                                  const float* __restrict__ grad_loss, const int* __restrict__ idx,
                                                  const float* __restrict__ p, int K, __bf16* __restrict__ G) {
  const int r = blockIdx.x;
  const int t = c0 + r;
  __bf16* g = G + (long long)r * v_pad;
  const bool live = r < rows && (mask == nullptr || mask[t] != 0);
  if (!live) {
    for (int v = threadIdx.x; v < v_pad; v += kT) g[v] = (__bf16)0.f;
    return;
  }
  const int nv = ctrl->n_valid;
  const float gw = nv > 0 ? grad_loss[0] / (float)nv : 0.f;
  const float coef = gw * S[t];
  const float* z = Z + (long long)r * ldz;
  const float shift = kDense ? 0.f : lse[t];
  for (int v = threadIdx.x; v < v_pad; v += kT) {
    float x = 0.f;
    if (v < V) {
      x = coef * exp_fast(z[v] - shift);
      if constexpr (kDense) x -= gw * P[(long long)r * ldz + v];
    }
    g[v] = (__bf16)x;
  }
  if constexpr (!kDense) {
    __syncthreads();  // the elementwise values above, then the teacher entries over them
    for (int k = threadIdx.x; k < K; k += kT) {
      const int v = idx[(long long)t * K + k];
      const float pk = p[(long long)t * K + k];
      if (v >= 0 && v < V && pk > 0.f) g[v] = (__bf16)(coef * exp_fast(z[v] - shift) - gw * pk);
    }
  }
}

}  // namespace

void launch_row_stats(const float* Z, long long ldz, int V, int rows, float2* part, hipStream_t s) {
  if (rows > 0) row_stats_kernel<<<rows, kT, 0, s>>>(Z, ldz, V, part);
}

void launch_log_softmax(float* Z, long long ldz, int V, int rows, int c0, float* lse, hipStream_t s) {
  if (rows > 0) log_softmax_kernel<<<rows, kT, 0, s>>>(Z, ldz, V, c0, lse);
}

void launch_teacher_grid(float* P, long long ldz, int V, int rows, int c0, const int* idx, const float* p,
                         const uint8_t* mask, int K, hipStream_t s) {
  if (rows > 0) teacher_grid_kernel<<<rows, kT, 0, s>>>(P, ldz, V, c0, idx, p, mask, K);
}

void launch_dense_kl(const float* P, const float* LQ, long long ldz, int V, int rows, int c0, const uint8_t* mask,
                     float* row_kl, hipStream_t s) {
  if (rows > 0) dense_kl_kernel<<<rows, kT, 0, s>>>(P, LQ, ldz, V, c0, mask, row_kl);
}

void launch_gather(const float* Z, long long ldz, int rows, int c0, const int* idx, const uint8_t* mask, int K,
                   int V, float* g, hipStream_t s) {
  const long long work = (long long)rows * K;
  if (work > 0) gather_kernel<<<(unsigned)((work + kT - 1) / kT), kT, 0, s>>>(Z, ldz, rows, c0, idx, mask, K, V, g);
}

void launch_grad_from_grid(bool dense, const float* Z, const float* P, long long ldz, int V, int v_pad, int rows,
                           int c_pad, int c0, const float* lse, const float* S, const uint8_t* mask,
                           const Ctrl* ctrl, const float* grad_loss, const int* idx, const float* p, int K,
                           void* G, hipStream_t s) {
  if (c_pad <= 0) return;
  if (dense)
    grad_kernel<true><<<c_pad, kT, 0, s>>>(Z, P, ldz, V, v_pad, rows, c0, lse, S, mask, ctrl, grad_loss, idx, p,
                                           K, static_cast<__bf16*>(G));
  else
    grad_kernel<false><<<c_pad, kT, 0, s>>>(Z, P, ldz, V, v_pad, rows, c0, lse, S, mask, ctrl, grad_loss, idx, p,
                                            K, static_cast<__bf16*>(G));
}

}  // namespace kd
