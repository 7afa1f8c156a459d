// Memory-bound kernels of the kdloss path: teacher preparation, teacher-hit
// bucketing, log-sum-exp merge with the per-row KL, the deterministic loss
// reduction, padded transposes and the split-K reduction of dH.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kd_internal.h"

namespace kd {
namespace {

constexpr float kNegInf = -__builtin_inff();

// Butterfly sum / max over the 64 lanes, every lane ending with the result,
// through register-only cross-lane moves instead of the LDS crossbar: quad
// permutes for partners i ^ 1 and i ^ 2, then the mirrored lane of the other
// quad of each 8 (row_half_mirror) and of the other 8 of each 16
// (row_mirror), then swaps of 16-lane rows and of 32-lane halves.  After each
// step every lane of a group holds the same value, so the partner taken from
// the other group has the value of lane i ^ o: the result is that of the xor
// butterfly (v op= v[i ^ o], o = 1 .. 32) bit for bit.
template <class Op>
__device__ inline float wave_reduce(float v, Op op) {
  auto dpp = [](float x, int ctrl) {
    switch (ctrl) {  // the control word must be a constant
      case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
      case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    }
  };
  v = op(v, dpp(v, 0xB1));   // quad_perm [1, 0, 3, 2]: lane i ^ 1
  v = op(v, dpp(v, 0x4E));   // quad_perm [2, 3, 0, 1]: lane i ^ 2
  v = op(v, dpp(v, 0x141));  // row_half_mirror: the other quad of the 8
  v = op(v, dpp(v, 0x140));  // row_mirror: the other 8 of the 16
  // (the swaps' results are copied to scalars first: a bit_cast applied to a
  // vector element reads element 0 with this compiler)
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 0 <-> 1, 2 <-> 3
  const unsigned a16 = r16[0], b16 = r16[1];
  v = op(__builtin_bit_cast(float, a16), __builtin_bit_cast(float, b16));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);  // halves
  const unsigned a32 = r32[0], b32 = r32[1];
  return op(__builtin_bit_cast(float, a32), __builtin_bit_cast(float, b32));
}

__device__ inline float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

__device__ inline float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
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

// Exclusive scan over the kWaves wavefronts of a workgroup (fixed order);
// *total receives the sum.  sh: kWaves ints of LDS.
template <int kWaves>
__device__ inline int block_exclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    base += w < wave ? sh[w] : 0;
    all += sh[w];
  }
  *total = all;
  __syncthreads();
  return base + incl - v;
}

// Slots of the per-wavefront table that detects repeated ids in a row of at
// most 128 entries (load factor <= 1/2).
constexpr int kDupSlots = 256;

// For one row of more than 128 entries (ids[0..K), p[0..K) as stored, p_of(k)
// recomputes p bitwise): where an id occurs more than once, p at its first
// occurrence becomes the sum of its occurrences' p in k order and p at the
// others becomes 0.  Every entry is compared with every other one.  Ids < 0
// or >= V are left alone.  Called by a whole wavefront.
template <class PK>
__device__ inline void resolve_repeated_ids(const int* ids, int K, int V, float* p, PK&& p_of) {
  const int lane = threadIdx.x & 63;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int k = k0 + lane;
    const int v = k < K ? ids[k] : -1;
    int f = k, n_same = 0;
    float sum = 0.f;
    for (int kq = 0; kq < K; kq += 64) {
      const int wv = kq + lane < K ? ids[kq + lane] : -1;
      const float pv = kq + lane < K ? p_of(kq + lane) : 0.f;
      const int here = min(64, K - kq);
      for (int u = 0; u < here; ++u) {
        const float pu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), u));
        if (__builtin_amdgcn_readlane(wv, u) == v) {
          ++n_same;
          f = min(f, kq + u);
          sum += pu;
        }
      }
    }
    if (v >= 0 && v < V && n_same > 1) p[k] = f == k ? sum : 0.f;
  }
}

// The same for a row whose K <= 128 entries sit in registers: entry k = lane
// in (v0, p0), entry 64 + lane in (v1, p1); slots past K hold id -1.  A table
// of kDupSlots ids in LDS detects a repeat (an insertion that finds its own id
// already there); only rows with one take the pairwise pass in k order.
__device__ inline void resolve_repeated_ids_regs(int v0, int v1, int V, float& p0, float& p1, int* t_id) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < kDupSlots; i += 64) t_id[i] = -1;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  bool dup = false;
  auto insert = [&](int v) {
    if (v < 0 || v >= V) return;
    int h = (int)(((unsigned)v * 2654435761u) >> 24);
    for (;;) {
      const int old = atomicCAS(&t_id[h], -1, v);
      if (old == -1) break;
      if (old == v) {
        dup = true;
        break;
      }
      h = (h + 1) & (kDupSlots - 1);
    }
  };
  insert(v0);
  insert(v1);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the table is cleared for the next row after this
  if (!__any(dup)) return;
  float np[2] = {p0, p1};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int v = c ? v1 : v0, k = 64 * c + lane;
    int f = k, n_same = 0;
    float sum = 0.f;
#pragma unroll
    for (int cq = 0; cq < 2; ++cq) {
      const int wv = cq ? v1 : v0;
      const float pv = cq ? p1 : p0;
      for (int u = 0; u < 64; ++u) {
        if (__builtin_amdgcn_readlane(wv, u) == v) {
          ++n_same;
          f = min(f, 64 * cq + u);
          sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), u));
        }
      }
    }
    if (v >= 0 && v < V && n_same > 1) np[c] = f == k ? sum : 0.f;
  }
  p0 = np[0];
  p1 = np[1];
}

// One workgroup (kBucketWaves wavefronts) per 64-row block.  Each wavefront
// takes one row at a time: renormalises the teacher's K log-values (the
// offline top-K cache of the blog's "Two systems changes"), computes
// p = exp(l), S = sum p and E = sum p*l (0*log 0 := 0), stores p (for an id
// the row repeats: the sum of its occurrences' p at the first one, 0 at the
// others), and counts the row's ids per vocabulary tile in LDS.  The counts
// are then scanned into this block's bucket offsets and every entry is placed
// in its bucket with LDS cursors.  Masked rows are skipped entirely; ids >= V
// set the range flag and are dropped; ids < 0 are padding (probability 0,
// outside the renormalisation).  The log-values are divided by the
// temperature (inv_tau = 1 / tau) before the renormalisation.
constexpr int kBucketWaves = 8;
constexpr int kBucketThreads = 64 * kBucketWaves;
__global__ __launch_bounds__(kBucketThreads) void teacher_bucket_kernel(
    const float* __restrict__ logp, const int* __restrict__ idx, const uint8_t* __restrict__ mask,
    int n, int K, int V, int n_vt, float inv_tau, float* __restrict__ p, float* __restrict__ S,
    float* __restrict__ E, int* __restrict__ hit_off, Hit* __restrict__ hits, Ctrl* ctrl) {
  extern __shared__ int cnt[];  // n_vt + 1 counters (then cursors), then the repeated-id tables
  __shared__ int sh[kBucketWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x;
  const int row_lo = rb * ROW_BLOCK, row_hi = min(row_lo + ROW_BLOCK, n);
  const int n_ct = n_vt + 1;
  int* const dup_tab = cnt + n_ct;  // kBucketWaves x kDupSlots
  for (int j = tid; j < n_ct; j += kBucketThreads) cnt[j] = 0;
  __syncthreads();

  int live_rows = 0;
  bool bad = false;
  // K <= 128: the rows of a wavefront (kRows of them) are loaded into
  // registers at once (entries lane and 64 + lane of each) and stay there
  // until placement, so the rows' loads overlap instead of running one after
  // another.
  constexpr int kRows = ROW_BLOCK / kBucketWaves;
  const bool regs = K <= 128;
  int rv0[kRows], rv1[kRows];
  float rp0[kRows], rp1[kRows];
  if (regs) {
    bool live[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = row_lo + wave + kBucketWaves * r;
      const bool in = row < row_hi;
      const long long base = (long long)row * K;
      rv0[r] = in && lane < K ? idx[base + lane] : -1;
      rv1[r] = in && lane + 64 < K ? idx[base + 64 + lane] : -1;
      rp0[r] = in && lane < K ? logp[base + lane] : 0.f;
      rp1[r] = in && lane + 64 < K ? logp[base + 64 + lane] : 0.f;
      live[r] = in && (mask == nullptr || mask[row] != 0);
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = row_lo + wave + kBucketWaves * r;
      if (row >= row_hi) continue;
      const long long base = (long long)row * K;
      if (!live[r]) {
        if (lane < K) p[base + lane] = 0.f;
        if (lane + 64 < K) p[base + 64 + lane] = 0.f;
        if (lane == 0) {
          S[row] = 0.f;
          E[row] = 0.f;
        }
        rv0[r] = rv1[r] = -1;  // nothing to place
        continue;
      }
      ++live_rows;
      // the same arithmetic, in the same order, as the general path below
      const float x0 = rv0[r] < 0 ? kNegInf : rp0[r] * inv_tau;
      const float x1 = rv1[r] < 0 ? kNegInf : rp1[r] * inv_tau;
      float mx = kNegInf;
      if (lane < K) mx = fmaxf(mx, x0);
      if (lane + 64 < K) mx = fmaxf(mx, x1);
      mx = wave_max(mx);
      float se = 0.f;
      if (lane < K) se += expf(x0 - mx);
      if (lane + 64 < K) se += expf(x1 - mx);
      se = wave_sum(se);
      const float lam = mx + logf(se);
      float sp = 0.f, e = 0.f, p0 = 0.f, p1 = 0.f;
      if (lane < K) {
        const float l = x0 - lam;
        p0 = expf(l);
        sp += p0;
        e += p0 > 0.f ? p0 * l : 0.f;
      }
      if (lane + 64 < K) {
        const float l = x1 - lam;
        p1 = expf(l);
        sp += p1;
        e += p1 > 0.f ? p1 * l : 0.f;
      }
      const int v0 = rv0[r], v1 = rv1[r];
      if (v0 >= 0 && v0 < V) atomicAdd(&cnt[v0 / TILE_V], 1);
      else if (v0 >= V) bad = true;
      if (v1 >= 0 && v1 < V) atomicAdd(&cnt[v1 / TILE_V], 1);
      else if (v1 >= V) bad = true;
      sp = wave_sum(sp);
      e = wave_sum(e);
      if (lane == 0) {
        S[row] = sp;
        E[row] = e;
      }
      resolve_repeated_ids_regs(v0, v1, V, p0, p1, dup_tab + wave * kDupSlots);
      if (lane < K) p[base + lane] = p0;
      if (lane + 64 < K) p[base + 64 + lane] = p1;
      rp0[r] = p0;
      rp1[r] = p1;
    }
  } else
  for (int row = row_lo + wave; row < row_hi; row += kBucketWaves) {
    const long long base = (long long)row * K;
    if (mask != nullptr && mask[row] == 0) {
      for (int k = lane; k < K; k += 64) p[base + k] = 0.f;
      if (lane == 0) {
        S[row] = 0.f;
        E[row] = 0.f;
      }
      continue;
    }
    ++live_rows;
    // softened log-value of entry k; padding entries (id < 0) count as -inf
    auto a_of = [&](int k) { return idx[base + k] < 0 ? kNegInf : logp[base + k] * inv_tau; };
    float mx = kNegInf;
    for (int k = lane; k < K; k += 64) mx = fmaxf(mx, a_of(k));
    mx = wave_max(mx);
    float se = 0.f;
    for (int k = lane; k < K; k += 64) se += expf(a_of(k) - mx);
    se = wave_sum(se);
    const float lam = mx + logf(se);
    float sp = 0.f, e = 0.f;
    for (int k = lane; k < K; k += 64) {
      const float l = a_of(k) - lam;
      const float pk = expf(l);
      p[base + k] = pk;
      sp += pk;
      e += pk > 0.f ? pk * l : 0.f;
      const int v = idx[base + k];
      if (v >= 0 && v < V)
        atomicAdd(&cnt[v / TILE_V], 1);
      else if (v >= V)
        bad = true;
    }
    sp = wave_sum(sp);
    e = wave_sum(e);
    if (lane == 0) {
      S[row] = sp;
      E[row] = e;
    }
    // Repeated ids.  The backward's scatter subtracts each entry's p from the
    // accumulator of (row, id), and entries reach it in the order of their
    // teacher-hit bucket, which the LDS cursors below make arbitrary; a
    // repeated id would put several subtractions on one accumulator in that
    // order.  So the first occurrence of an id keeps the sum of the p of all
    // its occurrences (added in k order) and the later ones keep 0: entries
    // of distinct (row, id) touch distinct accumulators and the result no
    // longer depends on the bucket order.  The forward's sum of p * g is the
    // same sum (repeated ids share one logit g); S and E above use every p.
    resolve_repeated_ids(idx + base, K, V, p + base, [&](int k) {
      return expf(a_of(k) - lam);  // bitwise the p stored above
    });
  }
  if (lane == 0 && live_rows > 0) atomicAdd(&ctrl->n_valid, live_rows);
  if (__any(bad) && lane == 0) ctrl->range_error = 1;
  __syncthreads();

  // Exclusive scan of the n_vt + 1 counters (the last one is 0, so it ends as
  // the block's total); thread t owns a contiguous run of them.
  const int per = (n_ct + kBucketThreads - 1) / kBucketThreads;
  const int j0 = min(tid * per, n_ct), j1 = min(j0 + per, n_ct);
  int run = 0;
  for (int j = j0; j < j1; ++j) run += cnt[j];
  int total;
  run = block_exclusive_scan<kBucketWaves>(run, sh, &total);
  const int hit_base = rb * ROW_BLOCK * K;
  int* off = hit_off + (long long)rb * n_ct;
  for (int j = j0; j < j1; ++j) {
    const int c = cnt[j];
    cnt[j] = run;
    off[j] = hit_base + run;
    run += c;
  }
  __syncthreads();

  // Placement.  Register path: ids and p (after the repeated-id pass) from
  // registers; rows past the block end and masked rows hold id -1.
  if (regs) {
    auto place = [&](int row, int k, int v, float pk) {
      if (v >= 0 && v < V) {
        const int pos = atomicAdd(&cnt[v / TILE_V], 1);
        Hit h;
        h.row = row;
        h.k = k;
        h.v = v;
        h.p = pk;
        hits[hit_base + pos] = h;
      }
    };
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = row_lo + wave + kBucketWaves * r;
      place(row, lane, rv0[r], rp0[r]);
      place(row, 64 + lane, rv1[r], rp1[r]);
    }
    return;
  }
  // General path: p is re-read from memory this workgroup wrote before the barrier.
  for (int row = row_lo + wave; row < row_hi; row += kBucketWaves) {
    if (mask != nullptr && mask[row] == 0) continue;
    const long long base = (long long)row * K;
    for (int k = lane; k < K; k += 64) {
      const int v = idx[base + k];
      if (v >= 0 && v < V) {
        const int pos = atomicAdd(&cnt[v / TILE_V], 1);
        Hit h;
        h.row = row;
        h.k = k;
        h.v = v;
        h.p = p[base + k];
        hits[hit_base + pos] = h;
      }
    }
  }
}

// 32 chunk rows per workgroup, 32 slices per row (1024 threads, so enough
// loads are in flight): slice s merges the per-vocabulary-tile (max, sum-exp)
// partials j = s, s+32, ... and the teacher terms k = s, s+32, ...; the slices
// are then combined in slice order.  The
// merge order depends only on the number of vocabulary tiles, so LSE and KL do
// not depend on the chunk size.  The partials are of the softened logits
// z / tau, so LSE_t is that of z / tau, and
// KL_t = tau^2 (E_t - sum_k p_k g_k / tau + S_t * LSE_t).
constexpr int kKlRows = 32, kKlSlices = 32;
__global__ __launch_bounds__(kKlRows * kKlSlices) void lse_kl_kernel(const float2* __restrict__ part, int ld_part,
                                                     int n_vt, int c0, int rows,
                                                     const float* __restrict__ p,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ S,
                                                     const float* __restrict__ E,
                                                     const uint8_t* __restrict__ mask, int K,
                                                     float tau, float* __restrict__ lse,
                                                     float* __restrict__ row_kl) {
  __shared__ float2 red[kKlSlices][kKlRows];
  __shared__ float dred[kKlSlices][kKlRows];
  const int rl = threadIdx.x % kKlRows, sl = threadIdx.x / kKlRows;
  const int r = blockIdx.x * kKlRows + rl;
  const bool ok = r < rows;
  const int t = c0 + r;
  float2 acc = make_float2(kNegInf, 0.f);
  if (ok) {
    int j = sl;
    for (; j + 3 * kKlSlices < n_vt; j += 4 * kKlSlices) {
      const float2 a = part[(long long)j * ld_part + r];
      const float2 b = part[(long long)(j + kKlSlices) * ld_part + r];
      const float2 c = part[(long long)(j + 2 * kKlSlices) * ld_part + r];
      const float2 d = part[(long long)(j + 3 * kKlSlices) * ld_part + r];
      acc = lse_merge(acc, a);
      acc = lse_merge(acc, b);
      acc = lse_merge(acc, c);
      acc = lse_merge(acc, d);
    }
    for (; j < n_vt; j += kKlSlices) acc = lse_merge(acc, part[(long long)j * ld_part + r]);
  }
  float dot = 0.f;
  const bool live = ok && (mask == nullptr || mask[t] != 0);
  if (live) {
    const long long base = (long long)t * K;
    for (int k = sl; k < K; k += kKlSlices) {
      const float pk = p[base + k];
      dot += pk > 0.f ? pk * g[base + k] : 0.f;
    }
  }
  red[sl][rl] = acc;
  dred[sl][rl] = dot;
  __syncthreads();
  if (sl == 0 && ok) {
    float2 m = red[0][rl];
    float dsum = dred[0][rl];
#pragma unroll
    for (int q = 1; q < kKlSlices; ++q) {
      m = lse_merge(m, red[q][rl]);
      dsum += dred[q][rl];
    }
    const float L = m.x + logf(m.y);
    lse[t] = L;
    row_kl[t] = live ? tau * tau * (E[t] - dsum / tau + S[t] * L) : 0.f;
  }
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

// out[c][r] = in[r][c] for r < rows, 0 for rows <= r < rows_pad.  64 x 64
// tiles; rows of the tile move as 16-byte vectors in both directions (W of
// element size es: 16/es elements per vector), through an LDS tile padded by
// one 4-byte word per row.
template <typename E>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const E* __restrict__ in, int rows,
                                                            int cols, long long ld_in,
                                                            E* __restrict__ out, int rows_pad,
                                                            long long ld_out) {
  constexpr int EPV = 16 / sizeof(E);          // elements per 16-byte vector
  constexpr int VPR = 64 / EPV;                // vectors per 64-element tile row
  constexpr int PITCH = 64 + 4 / sizeof(E);    // tile row pitch in elements
  __shared__ E tile[64 * PITCH];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const bool vec_in = (ld_in % EPV) == 0 && c0 + 64 <= cols;
#pragma unroll
  for (int q = tid; q < 64 * VPR; q += 256) {
    const int i = q / VPR, cv = (q % VPR) * EPV;
    const int r = r0 + i;
    E v[EPV];
    if (r < rows && vec_in) {
      *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(in + (long long)r * ld_in + c0 + cv);
    } else {
#pragma unroll
      for (int u = 0; u < EPV; ++u) v[u] = (r < rows && c0 + cv + u < cols) ? in[(long long)r * ld_in + c0 + cv + u] : E(0);
    }
#pragma unroll
    for (int u = 0; u < EPV; ++u) tile[i * PITCH + cv + u] = v[u];
  }
  __syncthreads();
  const bool vec_out = (ld_out % EPV) == 0 && r0 + 64 <= rows_pad;
#pragma unroll
  for (int q = tid; q < 64 * VPR; q += 256) {
    const int cl = q / VPR, rv = (q % VPR) * EPV;
    const int c = c0 + cl;
    if (c >= cols) continue;
    E v[EPV];
#pragma unroll
    for (int u = 0; u < EPV; ++u) v[u] = tile[(rv + u) * PITCH + cl];
    if (vec_out) {
      *reinterpret_cast<uint4*>(out + (long long)c * ld_out + r0 + rv) = *reinterpret_cast<const uint4*>(v);
    } else {
#pragma unroll
      for (int u = 0; u < EPV; ++u)
        if (r0 + rv + u < rows_pad) out[(long long)c * ld_out + r0 + rv + u] = v[u];
    }
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

void launch_teacher_bucket(const float* logp, const int* idx, const uint8_t* mask, int n, int K,
                           int V, float inv_tau, float* p, float* S, float* E, int* hit_off,
                           Hit* hits, Ctrl* ctrl, hipStream_t s) {
  const int n_vt = (V + TILE_V - 1) / TILE_V;
  const int n_rb = (n + ROW_BLOCK - 1) / ROW_BLOCK;
  const size_t lds = (size_t(n_vt + 1) + kBucketWaves * kDupSlots) * sizeof(int);
  teacher_bucket_kernel<<<n_rb, kBucketThreads, lds, s>>>(logp, idx, mask, n, K, V, n_vt, inv_tau, p, S, E,
                                               hit_off, hits, ctrl);
}

void launch_lse_kl(const float2* part, int ld_part, int n_vt, int c0, int rows, const float* p,
                   const float* g, const float* S, const float* E, const uint8_t* mask, int K,
                   float tau, float* lse, float* row_kl, hipStream_t s) {
  lse_kl_kernel<<<(rows + kKlRows - 1) / kKlRows, kKlRows * kKlSlices, 0, s>>>(part, ld_part, n_vt, c0, rows, p, g,
                                                                S, E, mask, K, tau, lse, row_kl);
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
