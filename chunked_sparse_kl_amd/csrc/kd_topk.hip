// Teacher top-K cache builder: the per-row threshold and the final selection.
//
// The cache the pages describe keeps, for every position, the K most likely
// teacher tokens and their values (Hugging Face blog "Making Knowledge
// Distillation Cheap Enough to Run at Scale", section "Two systems changes";
// aimodeling.com article, section "First cut: remove the teacher from the
// training loop").  The builder never stores a row's logits:
//   1. a GEMM pass gives per (row, 256-wide vocabulary tile) the maximum and
//      sum of exp(z - max) (the forward statistics epilogue);
//   2. topk_threshold_kernel: LSE_t from those partials, and thr_t = the K-th
//      largest tile maximum.  K distinct logits (the tile maxima) are >= thr_t,
//      so the K-th largest logit is >= thr_t and every top-K logit passes;
//   3. a second, bitwise identical GEMM pass appends every logit >= thr_t to
//      row t's candidate list (typically a few hundred entries);
//   4. topk_select_kernel: the K candidates with the largest logits, ties by
//      increasing id, in decreasing order, written as (id, z - LSE_t).
// Selection uses 64-bit keys (~ord(z) << 32 | id): ascending keys are
// decreasing logits, equal logits by increasing id, and keys are unique.
#include "kd_internal.h"

namespace kd {
namespace {

constexpr float kNegInf = -__builtin_inff();

// Order-preserving map of a (non-NaN) float to an unsigned integer.
__device__ inline unsigned ord_f32(float f) {
  const unsigned u = __builtin_bit_cast(unsigned, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float unord_f32(unsigned u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__device__ inline float2 merge_max_sum(float2 a, float2 b) {
  const float m = fmaxf(a.x, b.x);
  if (m == kNegInf) return make_float2(kNegInf, 0.f);
  return make_float2(m, a.y * __expf(a.x - m) + b.y * __expf(b.x - m));
}

// The rank-th smallest (1-based) of the c keys load(i), i < c: most
// significant digit first radix select, 8-bit digits.  All 256 threads of
// the workgroup call it with the same arguments; rank <= c.
template <typename Key, class Load>
__device__ Key kth_smallest(int c, int rank, const Load& load, unsigned* hist, int* sel) {
  constexpr int kBits = 8 * (int)sizeof(Key);
  const int tid = threadIdx.x;
  Key prefix = 0;
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    const Key hi_mask = shift + 8 >= kBits ? Key(0) : (~Key(0) << (shift + 8));
    for (int i = tid; i < c; i += 256) {
      const Key k = load(i);
      if ((k & hi_mask) == prefix) atomicAdd(&hist[(unsigned)(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned below = 0;
      int d = 0;
      for (; d < 255; ++d) {
        if (below + hist[d] >= (unsigned)rank) break;
        below += hist[d];
      }
      sel[0] = d;
      sel[1] = rank - (int)below;
    }
    __syncthreads();
    prefix |= Key(sel[0]) << shift;
    rank = sel[1];
    __syncthreads();
  }
  return prefix;
}

// Ascending bitonic sort of p (a power of two) keys in LDS by 256 threads.
template <typename Key>
__device__ void bitonic_sort(Key* a, int p) {
  for (int k = 2; k <= p; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < p; i += 256) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const Key x = a[i], y = a[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// One workgroup per chunk row r (dynamic LDS: n_vt tile maxima).
__global__ __launch_bounds__(256) void topk_threshold_kernel(const float2* __restrict__ part,
                                                             int ld_part, int n_vt, int K,
                                                             float* __restrict__ lse,
                                                             float* __restrict__ thr) {
  extern __shared__ unsigned tile_key[];  // ~ord(max of tile j)
  __shared__ float2 red[256];
  __shared__ unsigned hist[256];
  __shared__ int sel[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  float2 acc = make_float2(kNegInf, 0.f);
  for (int j = tid; j < n_vt; j += 256) {
    const float2 pj = part[(long long)j * ld_part + r];
    tile_key[j] = ~ord_f32(pj.x);
    acc = merge_max_sum(acc, pj);
  }
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {  // fixed-order tree
    if (tid < s) red[tid] = merge_max_sum(red[tid], red[tid + s]);
    __syncthreads();
  }
  float t = kNegInf;
  if (n_vt >= K) {
    const unsigned key = kth_smallest<unsigned>(n_vt, K, [&](int i) { return tile_key[i]; }, hist, sel);
    t = unord_f32(~key);
  }
  if (tid == 0) {
    lse[r] = red[0].x + logf(red[0].y);
    thr[r] = t;
  }
}

// One workgroup per chunk row r (dynamic LDS: p >= K keys, a power of two).
__global__ __launch_bounds__(256) void topk_select_kernel(const int2* __restrict__ cand, int cap,
                                                          const int* __restrict__ cnt,
                                                          const float* __restrict__ lse, int K, int p,
                                                          int c0, int* __restrict__ out_idx,
                                                          float* __restrict__ out_logp, Ctrl* ctrl) {
  extern __shared__ unsigned long long sk[];
  __shared__ unsigned hist[256];
  __shared__ int sel[2];
  __shared__ int n_sel;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int total = cnt[r];
  const int c = min(total, cap);
  if (tid == 0 && total > cap) atomicAdd(&ctrl->overflow_rows, 1);
  const int2* cr = cand + (long long)r * cap;
  auto key_of = [&](int i) -> unsigned long long {
    const int2 e = cr[i];
    return ((unsigned long long)~ord_f32(__builtin_bit_cast(float, e.y)) << 32) | (unsigned)e.x;
  };
  const int want = min(K, c);
  unsigned long long kth = 0ull;
  if (want > 0) kth = kth_smallest<unsigned long long>(c, want, key_of, hist, sel);
  for (int i = tid; i < p; i += 256) sk[i] = ~0ull;
  if (tid == 0) n_sel = 0;
  __syncthreads();
  if (want > 0) {
    for (int i = tid; i < c; i += 256) {
      const unsigned long long k = key_of(i);
      if (k <= kth) {
        const int q = atomicAdd(&n_sel, 1);
        if (q < p) sk[q] = k;
      }
    }
  }
  __syncthreads();
  bitonic_sort(sk, p);
  const float L = lse[r];
  const long long o = (long long)(c0 + r) * K;
  for (int k = tid; k < K; k += 256) {
    const unsigned long long key = sk[k];
    if (key == ~0ull) {  // fewer than K candidates (only with NaN logits): padding
      out_idx[o + k] = -1;
      out_logp[o + k] = kNegInf;
    } else {
      out_idx[o + k] = (int)(unsigned)key;
      out_logp[o + k] = unord_f32(~(unsigned)(key >> 32)) - L;
    }
  }
}

}  // namespace

void launch_topk_threshold(const float2* part, int ld_part, int n_vt, int K, int rows, float* lse,
                           float* thr, hipStream_t s) {
  topk_threshold_kernel<<<rows, 256, (size_t)n_vt * sizeof(unsigned), s>>>(part, ld_part, n_vt, K,
                                                                             lse, thr);
}

void launch_topk_select(const int2* cand, int cap, const int* cnt, const float* lse, int K, int rows,
                        int c0, int* out_idx, float* out_logp, Ctrl* ctrl, hipStream_t s) {
  int p = 1;
  while (p < K) p <<= 1;
  topk_select_kernel<<<rows, 256, (size_t)p * sizeof(unsigned long long), s>>>(
      cand, cap, cnt, lse, K, p, c0, out_idx, out_logp, ctrl);
}

}  // namespace kd
