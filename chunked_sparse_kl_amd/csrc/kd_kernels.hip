// Memory-bound kernels of the kdloss path: teacher preparation, teacher-hit
// bucketing, log-sum-exp merge with the per-row KL, the deterministic loss
// reduction, padded transposes and the split-K reduction of dH.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kd_internal.h"

namespace kd {
namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Merge of two (max, sum of exp(x - max)) pairs.
__device__ inline float2 lse_merge(float2 a, float2 b) {
  float m = fmaxf(a.x, b.x);
  if (m == kNegInf) return make_float2(kNegInf, 0.f);
  return make_float2(m, a.y * __expf(a.x - m) + b.y * __expf(b.x - m));
}

__global__ void fill_i32_kernel(int* p, long long count, int value) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long stride = (long long)gridDim.x * blockDim.x;
  for (; i < count; i += stride) p[i] = value;
}

// One wavefront per row.  Renormalises the teacher's K log-values (the offline
// top-K cache of the blog's "Two systems changes"), stores p = exp(l), S = sum p,
// E = sum p*l (0*log 0 := 0), counts unmasked rows and histograms the teacher
// ids by (vocabulary tile, row block).  Masked rows are skipped entirely.
__global__ __launch_bounds__(256) void teacher_prep_kernel(
    const float* __restrict__ logp, const int* __restrict__ idx, const uint8_t* __restrict__ mask,
    int n, int K, int V, float* __restrict__ p, float* __restrict__ S, float* __restrict__ E,
    int* __restrict__ counts, int n_rb, Ctrl* ctrl) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const long long base = (long long)row * K;
  const bool live = mask == nullptr || mask[row] != 0;
  if (!live) {
    for (int k = lane; k < K; k += 64) p[base + k] = 0.f;
    if (lane == 0) {
      S[row] = 0.f;
      E[row] = 0.f;
    }
    return;
  }
  float mx = kNegInf;
  for (int k = lane; k < K; k += 64) mx = fmaxf(mx, logp[base + k]);
  mx = wave_max(mx);
  float se = 0.f;
  for (int k = lane; k < K; k += 64) se += expf(logp[base + k] - mx);
  se = wave_sum(se);
  const float lam = mx + logf(se);
  float s = 0.f, e = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float l = logp[base + k] - lam;
    const float pk = expf(l);
    p[base + k] = pk;
    s += pk;
    e += pk > 0.f ? pk * l : 0.f;
  }
  s = wave_sum(s);
  e = wave_sum(e);
  if (lane == 0) {
    S[row] = s;
    E[row] = e;
    atomicAdd(&ctrl->n_valid, 1);
  }
  const int rb = row / ROW_BLOCK;
  bool bad = false;
  for (int k = lane; k < K; k += 64) {
    const int v = idx[base + k];
    if (v >= 0 && v < V)
      atomicAdd(&counts[(v / TILE_V) * n_rb + rb], 1);
    else
      bad = true;
  }
  if (__any(bad) && lane == 0) ctrl->range_error = 1;
}

// Block-level exclusive scan of 4096 ints (1024 threads x 4), deterministic.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanThreads * kScanItems;

__device__ inline int block_exclusive_scan(int v, int* sh_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh_waves[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      int t = sh_waves[w];
      sh_waves[w] = acc;
      acc += t;
    }
    *total = acc;
  }
  __syncthreads();
  int r = sh_waves[wave] + incl - v;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kScanThreads) void scan_tiles_kernel(const int* __restrict__ in, int n,
                                                                   int* __restrict__ tile_tot) {
  __shared__ int sh[kScanThreads / 64];
  __shared__ int tot;
  const long long b = (long long)blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) s += (b + i < n) ? in[b + i] : 0;
  block_exclusive_scan(s, sh, &tot);
  if (threadIdx.x == 0) tile_tot[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kScanThreads) void scan_totals_kernel(int* tile_tot, int n_tiles) {
  // exclusive scan in place of up to kScanTile tile totals (single block)
  __shared__ int sh[kScanThreads / 64];
  __shared__ int tot;
  int vals[kScanItems];
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const int j = threadIdx.x * kScanItems + i;
    vals[i] = j < n_tiles ? tile_tot[j] : 0;
    s += vals[i];
  }
  int run = block_exclusive_scan(s, sh, &tot);
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const int j = threadIdx.x * kScanItems + i;
    if (j < n_tiles) tile_tot[j] = run;
    run += vals[i];
  }
  if (threadIdx.x == 0) tile_tot[n_tiles] = tot;
}

__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(const int* __restrict__ in, int n,
                                                                  const int* __restrict__ tile_tot,
                                                                  int* __restrict__ out,
                                                                  int* __restrict__ cursor) {
  __shared__ int sh[kScanThreads / 64];
  __shared__ int tot;
  const long long b = (long long)blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int vals[kScanItems];
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    vals[i] = (b + i < n) ? in[b + i] : 0;
    s += vals[i];
  }
  int run = block_exclusive_scan(s, sh, &tot) + tile_tot[blockIdx.x];
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    if (b + i < n) {
      out[b + i] = run;
      cursor[b + i] = run;
    }
    run += vals[i];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) out[n] = tile_tot[gridDim.x];
}

// One wavefront per row: places every (row, k) of an unmasked row with a valid
// id into its (vocabulary tile, row block) bucket.
__global__ __launch_bounds__(256) void hit_scatter_kernel(const int* __restrict__ idx,
                                                          const float* __restrict__ p,
                                                          const uint8_t* __restrict__ mask, int n,
                                                          int K, int V, int n_rb,
                                                          int* __restrict__ cursor,
                                                          Hit* __restrict__ hits) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  if (mask != nullptr && mask[row] == 0) return;
  const long long base = (long long)row * K;
  const int rb = row / ROW_BLOCK;
  for (int k = lane; k < K; k += 64) {
    const int v = idx[base + k];
    if (v >= 0 && v < V) {
      const int pos = atomicAdd(&cursor[(v / TILE_V) * n_rb + rb], 1);
      Hit h;
      h.row = row;
      h.k = k;
      h.v = v;
      h.p = p[base + k];
      hits[pos] = h;
    }
  }
}

// One thread per chunk row: merges the per-vocabulary-tile (max, sum-exp)
// partials into the full-vocabulary LSE (fixed order, so the result does not
// depend on the chunk size), then KL_t = E_t - sum_k p_k g_k + S_t * LSE_t.
__global__ __launch_bounds__(256) void lse_kl_kernel(const float2* __restrict__ part, int ld_part,
                                                     int n_vt, int c0, int rows,
                                                     const float* __restrict__ p,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ S,
                                                     const float* __restrict__ E,
                                                     const uint8_t* __restrict__ mask, int K,
                                                     float* __restrict__ lse,
                                                     float* __restrict__ row_kl) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int t = c0 + r;
  float2 acc = make_float2(kNegInf, 0.f);
  int j = 0;
  for (; j + 4 <= n_vt; j += 4) {
    float2 a = part[(long long)(j + 0) * ld_part + r];
    float2 b = part[(long long)(j + 1) * ld_part + r];
    float2 c = part[(long long)(j + 2) * ld_part + r];
    float2 d = part[(long long)(j + 3) * ld_part + r];
    acc = lse_merge(acc, a);
    acc = lse_merge(acc, b);
    acc = lse_merge(acc, c);
    acc = lse_merge(acc, d);
  }
  for (; j < n_vt; ++j) acc = lse_merge(acc, part[(long long)j * ld_part + r]);
  const float L = acc.x + logf(acc.y);
  lse[t] = L;
  float kl = 0.f;
  if (mask == nullptr || mask[t] != 0) {
    const long long base = (long long)t * K;
    float dot = 0.f;
    for (int k = 0; k < K; ++k) {
      const float pk = p[base + k];
      dot += pk > 0.f ? pk * g[base + k] : 0.f;
    }
    kl = E[t] - dot + S[t] * L;
  }
  row_kl[t] = kl;
}

// Single block, fixed order: loss = sum_t row_kl[t] / N_valid (0 if none).
__global__ __launch_bounds__(1024) void loss_kernel(const float* __restrict__ row_kl, int n,
                                                    const Ctrl* ctrl, float* __restrict__ loss) {
  __shared__ double sh[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)row_kl[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int nv = ctrl->n_valid;
    loss[0] = nv > 0 ? (float)(sh[0] / (double)nv) : 0.f;
  }
}

// out[c][r] = in[r][c] for r < rows, 0 for rows <= r < rows_pad.  64x64 tiles.
template <typename E>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const E* __restrict__ in, int rows,
                                                            int cols, long long ld_in,
                                                            E* __restrict__ out, int rows_pad,
                                                            long long ld_out) {
  __shared__ E tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? in[(long long)r * ld_in + c] : E(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_pad) out[(long long)c * ld_out + r] = tile[tx][i];
  }
}

template <typename E>
__device__ inline E from_f32(float x);
template <>
__device__ inline float from_f32<float>(float x) { return x; }
template <>
__device__ inline __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// dH[r][j] = sum_s part[s][r][j] in fixed order, rounded to the output dtype.
template <typename E>
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* __restrict__ part, int splits,
                                                        long long split_stride, int rows, int d,
                                                        E* __restrict__ dH) {
  const long long total4 = (long long)rows * d / 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total4;
       i += (long long)gridDim.x * blockDim.x) {
    float4 acc = reinterpret_cast<const float4*>(part)[i];
    for (int s = 1; s < splits; ++s) {
      const float4 v = reinterpret_cast<const float4*>(part + s * split_stride)[i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    E* o = dH + i * 4;
    o[0] = from_f32<E>(acc.x);
    o[1] = from_f32<E>(acc.y);
    o[2] = from_f32<E>(acc.z);
    o[3] = from_f32<E>(acc.w);
  }
}

inline int grid_for(long long work, int per_block, int cap = 65536) {
  long long b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (int)b;
}

}  // namespace

void launch_fill_i32(int* p, long long count, int value, hipStream_t s) {
  if (count <= 0) return;
  fill_i32_kernel<<<grid_for(count, 256, 4096), 256, 0, s>>>(p, count, value);
}

void launch_teacher_prep(const float* logp, const int* idx, const uint8_t* mask, int n, int K,
                         int V, float* p, float* S, float* E, int* counts, int n_rb, Ctrl* ctrl,
                         hipStream_t s) {
  teacher_prep_kernel<<<(n + 3) / 4, 256, 0, s>>>(logp, idx, mask, n, K, V, p, S, E, counts, n_rb,
                                                  ctrl);
}

void launch_scan(const int* counts, int n_keys, int* offsets, int* cursor, int* tmp, hipStream_t s) {
  const int tiles = (n_keys + kScanTile - 1) / kScanTile;
  scan_tiles_kernel<<<tiles, kScanThreads, 0, s>>>(counts, n_keys, tmp);
  scan_totals_kernel<<<1, kScanThreads, 0, s>>>(tmp, tiles);
  scan_apply_kernel<<<tiles, kScanThreads, 0, s>>>(counts, n_keys, tmp, offsets, cursor);
}

void launch_hit_scatter(const int* idx, const float* p, const uint8_t* mask, int n, int K, int V,
                        int n_rb, int* cursor, Hit* hits, hipStream_t s) {
  hit_scatter_kernel<<<(n + 3) / 4, 256, 0, s>>>(idx, p, mask, n, K, V, n_rb, cursor, hits);
}

void launch_lse_kl(const float2* part, int ld_part, int n_vt, int c0, int rows, const float* p,
                   const float* g, const float* S, const float* E, const uint8_t* mask, int K,
                   float* lse, float* row_kl, hipStream_t s) {
  lse_kl_kernel<<<(rows + 255) / 256, 256, 0, s>>>(part, ld_part, n_vt, c0, rows, p, g, S, E, mask,
                                                   K, lse, row_kl);
}

void launch_loss(const float* row_kl, int n, const Ctrl* ctrl, float* loss, hipStream_t s) {
  loss_kernel<<<1, 1024, 0, s>>>(row_kl, n, ctrl, loss);
}

void launch_transpose_pad(DType t, const void* in, int rows, int cols, long long ld_in, void* out,
                          int rows_pad, long long ld_out, hipStream_t s) {
  dim3 grid((rows_pad + 63) / 64, (cols + 63) / 64);
  if (t == DType::BF16)
    transpose_pad_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(in), rows,
                                                        cols, ld_in, static_cast<uint16_t*>(out),
                                                        rows_pad, ld_out);
  else
    transpose_pad_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(in), rows, cols,
                                                     ld_in, static_cast<float*>(out), rows_pad,
                                                     ld_out);
}

void launch_dh_reduce(DType t, const float* part, int splits, long long split_stride, int rows,
                      int d, void* dH, hipStream_t s) {
  const long long work = (long long)rows * d / 4;
  if (work <= 0) return;
  const int grid = grid_for(work, 256, 8192);
  if (t == DType::BF16)
    dh_reduce_kernel<__bf16><<<grid, 256, 0, s>>>(part, splits, split_stride, rows, d,
                                                  static_cast<__bf16*>(dH));
  else
    dh_reduce_kernel<float><<<grid, 256, 0, s>>>(part, splits, split_stride, rows, d,
                                                 static_cast<float*>(dH));
}

}  // namespace kd
