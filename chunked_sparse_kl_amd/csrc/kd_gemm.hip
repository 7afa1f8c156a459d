// MFMA GEMM core of kdloss (gfx950) and its four epilogues.
//
// Every contraction of the path is written as  D[m][n] = sum_k A[m][k] * B[n][k]
// with both operands stored K-contiguous ("NT"), so one main loop serves all:
//   forward / recompute:  A = W [V][d],      B = H_c [C][d]     (D = logits^T)
//   dH:                   A = G [C][V],      B = W^T [d][V]     (split over V)
//   dW:                   A = G^T [V][C],    B = H_c^T [d][C]
// A 256-thread workgroup (4 wavefronts in a 2x2 grid) owns a 256 x BN tile;
// each wavefront owns 128 x BN/2 and accumulates it in 32x32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2f32 for fp32).  The
// K loop stages 128-byte rows of A and B through LDS, double buffered, with an
// XOR swizzle of the 16-byte chunks so that both the row-wise stores and the
// fragment loads are free of bank conflicts; the next K block is fetched into
// registers while the current one is multiplied.
//
// Accumulator layout of one 32x32 block (lane l, register e = 4*i + j):
//   row  = 8*i + 4*(l / 32) + j,   column = l % 32.
#include <hip/hip_runtime.h>

#include "kd_internal.h"

namespace kd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

constexpr int BM = 256;
constexpr int ROWB = 128;         // bytes per staged row of A or B (one K block)
constexpr int kThreads = 256;

template <typename T>
struct Traits;
template <>
struct Traits<__bf16> {
  static constexpr int BK = 64;   // K elements per block (128 bytes)
};
template <>
struct Traits<float> {
  static constexpr int BK = 32;
};

template <int BN>
struct Smem {
  static constexpr int kStage = (BM + BN) * ROWB;
  static constexpr int kBytes = 2 * kStage;
};

// LDS staging of epilogue values: 64 token slots x 256 vocab entries (fp32),
// row pitch padded to keep the 16-byte stores conflict free.
constexpr int kStgLd = BM + 4;

struct TileIdx {
  int tm, tn, split;
};

// Workgroups are dispatched round-robin over the 8 XCDs.  Give each XCD a
// contiguous range of tiles and walk it in groups of kGroupM A-tiles, so the
// workgroups resident on one XCD share A and B tiles in that XCD's L2.
template <int kGroupM>
__device__ inline TileIdx map_tile(int tiles_m, int tiles_n, int splits) {
  const int total = tiles_m * tiles_n * splits;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = total >> 3, rem = total & 7;
  const int lin = xcd * per + min(xcd, rem) + local;
  const int per_split = tiles_m * tiles_n;
  TileIdx t;
  t.split = lin / per_split;
  const int r = lin - t.split * per_split;
  const int span = kGroupM * tiles_n;
  const int group = r / span;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int w = r - group * span;
  t.tm = first_m + w % gsize;
  t.tn = w / gsize;
  return t;
}

template <typename T>
__device__ inline void mma_block(const uint4& a, const uint4& b, f32x16& acc);

template <>
__device__ inline void mma_block<__bf16>(const uint4& a, const uint4& b, f32x16& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <>
__device__ inline void mma_block<float>(const uint4& a, const uint4& b, f32x16& acc) {
  const f32x4 av = __builtin_bit_cast(f32x4, a);
  const f32x4 bv = __builtin_bit_cast(f32x4, b);
  // Lane (r, h) supplies k = 8s + 4h + e in instruction e, identically for A and B.
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[0], bv[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[1], bv[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[2], bv[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[3], bv[3], acc, 0, 0, 0);
}

struct Operand {
  const char* base;   // row 0, k 0
  long long ld;       // row pitch in bytes
  int rows;           // rows >= this read as zero
};

// Main loop: accumulates the tile (tm, tn) over K blocks [kb0, kb1).
template <typename T, int BN>
__device__ inline void gemm_mainloop(const Operand& A, const Operand& B, int k_elems, int tm, int tn,
                                     int kb0, int kb1, char* smem, f32x16 (&acc)[4][BN / 64]) {
  constexpr int BK = Traits<T>::BK;
  constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte chunk
  constexpr int A_LD = BM * 8 / kThreads;        // 16-byte loads per thread per K block
  constexpr int B_LD = BN * 8 / kThreads;
  constexpr int NBJ = BN / 64;
  constexpr int kStage = Smem<BN>::kStage;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;

  // Per-thread load slots: chunk q = i*256 + tid -> row q/8 = i*32 + tid/8 and
  // 16-byte chunk tid%8, the same chunk for every slot i of a thread.
  const int row0 = tid >> 3, c = tid & 7;
  const int kc = c * EPC;
  const int a_row = tm * BM + row0, b_row = tn * BN + row0;
  const char* a_src = A.base + (long long)a_row * A.ld + c * 16;
  const char* b_src = B.base + (long long)b_row * B.ld + c * 16;
  const long long a_step = 32 * A.ld, b_step = 32 * B.ld;
  const int dst0 = row0 * ROWB + ((c ^ (row0 & 7)) << 4);  // + i*32*ROWB

  uint4 ra[A_LD], rb[B_LD];
  auto gload = [&](int kb) {
    const bool k_ok = kb * BK + kc < k_elems;
    const long long off = (long long)kb * ROWB;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      ra[i] = (k_ok && a_row + 32 * i < A.rows)
                  ? *reinterpret_cast<const uint4*>(a_src + i * a_step + off)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      rb[i] = (k_ok && b_row + 32 * i < B.rows)
                  ? *reinterpret_cast<const uint4*>(b_src + i * b_step + off)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int st) {
    char* base = smem + st * kStage + dst0;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(base + i * 32 * ROWB) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      *reinterpret_cast<uint4*>(base + BM * ROWB + i * 32 * ROWB) = rb[i];
  };

  if (kb0 < kb1) {
    gload(kb0);
    lstore(0);
  }
  __syncthreads();
  const int a_row0 = (wr * 128 + r32) * ROWB;
  const int b_row0 = BM * ROWB + (wc * (BN / 2) + r32) * ROWB;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) & 1;
    const bool more = kb + 1 < kb1;
    if (more) gload(kb + 1);
    const char* S = smem + st * kStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = ((2 * s + h) ^ (r32 & 7)) << 4;
      uint4 fa[4], fb[NBJ];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        fa[bi] = *reinterpret_cast<const uint4*>(S + a_row0 + bi * 32 * ROWB + ch);
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj)
        fb[bj] = *reinterpret_cast<const uint4*>(S + b_row0 + bj * 32 * ROWB + ch);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) mma_block<T>(fa[bi], fb[bj], acc[bi][bj]);
    }
    if (more) lstore(st ^ 1);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ forward
// D[v][t] = z_{t,v}.  Per token: max and sum of exp(z - max) over this tile's
// vocabulary rows (-> one (max, sum) partial per vocabulary tile), then the
// logits at the token's teacher ids are copied out of an LDS-staged slice.
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void fwd_gemm_kernel(Operand A, Operand B, int k_elems,
                                                                int tiles_m, int tiles_n,
                                                                FwdEpilogue ep) {
  constexpr int BN = 256, NBJ = BN / 64;
  __shared__ __attribute__((aligned(16))) char smem[Smem<BN>::kBytes];
  const TileIdx ti = map_tile<4>(tiles_m, tiles_n, 1);
  f32x16 acc[4][NBJ];
  const int kb_end = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  gemm_mainloop<T, BN>(A, B, k_elems, ti.tm, ti.tn, 0, kb_end, smem, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, r32 = lane & 31, h = lane >> 5;
  const int v_base = ti.tm * BM + wr * 128 + 4 * h;  // + bi*32 + 8*i + j
  const bool full_v = (ti.tm + 1) * BM <= ep.V;

  // --- per-token (max, sum-exp) over this wavefront's 128 vocabulary rows
  float tmax[NBJ], tsum[NBJ];
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    float mx = kNegInf;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = v_base + bi * 32 + 8 * (e >> 2) + (e & 3);
        if (full_v || v < ep.V) mx = fmaxf(mx, acc[bi][bj][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sm = 0.f;
    if (mx != kNegInf) {
      const float mxs = mx * kLog2e;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int v = v_base + bi * 32 + 8 * (e >> 2) + (e & 3);
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[bi][bj][e], kLog2e, -mxs));
          if (full_v || v < ep.V) sm += x;
        }
    }
    sm += __shfl_xor(sm, 32, 64);
    tmax[bj] = mx;
    tsum[bj] = sm;
  }
  // --- merge the two vocabulary halves (wr = 0, 1) through LDS
  float2* red = reinterpret_cast<float2*>(smem);
  if (h == 0) {
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
      red[wr * BN + wc * 128 + bj * 32 + r32] = make_float2(tmax[bj], tsum[bj]);
  }
  __syncthreads();
  {
    const int n = ti.tn * BN + tid;  // one token per thread
    if (n < ep.rows) {
      const float2 a = red[tid], b = red[BN + tid];
      const float m = fmaxf(a.x, b.x);
      float s = 0.f;
      if (m != kNegInf) s = a.y * __builtin_amdgcn_exp2f((a.x - m) * kLog2e) +
                            b.y * __builtin_amdgcn_exp2f((b.x - m) * kLog2e);
      ep.part[(long long)ti.tm * ep.ld_part + n] = make_float2(m, s);
    }
  }

  // --- gather the logits at the teacher ids that fall in this tile
  const int row_lo = ep.c0 + ti.tn * BN;
  const int row_hi = ep.c0 + min(ti.tn * BN + BN, ep.rows);
  const int key0 = ti.tm * ep.n_rb;
  const int h_lo = ep.hit_off[key0 + row_lo / ROW_BLOCK];
  const int h_hi = ep.hit_off[key0 + (row_hi + ROW_BLOCK - 1) / ROW_BLOCK];
  if (h_lo >= h_hi) return;  // uniform over the workgroup
  float* stg = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int round = 0; round < NBJ; ++round) {
    __syncthreads();
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v4 = {acc[bi][round][4 * i + 0], acc[bi][round][4 * i + 1],
                    acc[bi][round][4 * i + 2], acc[bi][round][4 * i + 3]};
        *reinterpret_cast<f32x4*>(stg + (wc * 32 + r32) * kStgLd + wr * 128 + bi * 32 + 8 * i +
                                  4 * h) = v4;
      }
    __syncthreads();
    for (int x = h_lo + tid; x < h_hi; x += kThreads) {
      const int2 hk = ep.hits[x];
      const int nl = hk.x - row_lo;  // token within the tile
      if (nl < 0 || nl >= BN || ((nl >> 5) & 3) != round) continue;
      const long long gi = (long long)hk.x * ep.K + hk.y;
      const int vl = ep.idx[gi] - ti.tm * BM;
      ep.g[gi] = stg[((nl >> 7) * 32 + (nl & 31)) * kStgLd + vl];
    }
  }
}

// ------------------------------------------------------------------ recompute
// D[v][t] = z_{t,v} again; G_{t,v} = gw*S_t*q_{t,v} - gw*sum_k p_{t,k}[i_{t,k} = v]
// with gw = grad_loss * mask_t / N_valid, staged through LDS (fp32) where the
// scatter is applied, then rounded to T and written row-major (G) and
// transposed (G^T).
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void recompute_gemm_kernel(Operand A, Operand B,
                                                                      int k_elems, int tiles_m,
                                                                      int tiles_n,
                                                                      RecomputeEpilogue ep) {
  constexpr int BN = 256, NBJ = BN / 64;
  __shared__ __attribute__((aligned(16))) char smem[Smem<BN>::kBytes];
  const TileIdx ti = map_tile<4>(tiles_m, tiles_n, 1);
  f32x16 acc[4][NBJ];
  const int kb_end = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  gemm_mainloop<T, BN>(A, B, k_elems, ti.tm, ti.tn, 0, kb_end, smem, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, r32 = lane & 31, h = lane >> 5;
  const int v_base = ti.tm * BM + wr * 128 + 4 * h;
  const bool full_v = (ti.tm + 1) * BM <= ep.V;
  const int nv = ep.ctrl->n_valid;
  const float gw = nv > 0 ? ep.grad_loss[0] / (float)nv : 0.f;

#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    const int n = ti.tn * BN + wc * 128 + bj * 32 + r32;
    const int t = ep.c0 + n;
    const bool live = n < ep.rows && (ep.mask == nullptr || ep.mask[t] != 0);
    const float coef = live ? gw * ep.S[t] : 0.f;
    const float lse2 = live ? ep.lse[t] * kLog2e : 0.f;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = v_base + bi * 32 + 8 * (e >> 2) + (e & 3);
        const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[bi][bj][e], kLog2e, -lse2));
        acc[bi][bj][e] = (coef != 0.f && (full_v || v < ep.V)) ? coef * q : 0.f;
      }
  }

  const int row_lo = ep.c0 + ti.tn * BN;
  const int row_hi = ep.c0 + min(ti.tn * BN + BN, ep.rows);
  const int key0 = ti.tm * ep.n_rb;
  const int h_lo = row_lo < row_hi ? ep.hit_off[key0 + row_lo / ROW_BLOCK] : 0;
  const int h_hi = row_lo < row_hi ? ep.hit_off[key0 + (row_hi + ROW_BLOCK - 1) / ROW_BLOCK] : 0;
  float* stg = reinterpret_cast<float*>(smem);
  T* G = static_cast<T*>(ep.G);
  T* GT = static_cast<T*>(ep.GT);
  constexpr int EPC = 16 / sizeof(T);

#pragma unroll
  for (int round = 0; round < NBJ; ++round) {
    __syncthreads();
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v4 = {acc[bi][round][4 * i + 0], acc[bi][round][4 * i + 1],
                    acc[bi][round][4 * i + 2], acc[bi][round][4 * i + 3]};
        *reinterpret_cast<f32x4*>(stg + (wc * 32 + r32) * kStgLd + wr * 128 + bi * 32 + 8 * i +
                                  4 * h) = v4;
      }
    __syncthreads();
    for (int x = h_lo + tid; x < h_hi; x += kThreads) {
      const int2 hk = ep.hits[x];
      const int nl = hk.x - row_lo;
      if (nl < 0 || nl >= BN || ((nl >> 5) & 3) != round) continue;
      const long long gi = (long long)hk.x * ep.K + hk.y;
      const int vl = ep.idx[gi] - ti.tm * BM;
      atomicAdd(&stg[((nl >> 7) * 32 + (nl & 31)) * kStgLd + vl], -gw * ep.p[gi]);
    }
    __syncthreads();
    // G rows: 64 token slots x 256 vocab, EPC elements per 16-byte store.
    constexpr int kRowChunks = BM / EPC;
#pragma unroll
    for (int it = 0; it < 64 * kRowChunks / kThreads; ++it) {
      const int q = it * kThreads + tid;
      const int slot = q / kRowChunks, c = q % kRowChunks;
      const int n = ti.tn * BN + (slot >> 5) * 128 + round * 32 + (slot & 31);
      const int v0 = ti.tm * BM + c * EPC;
      if (n < ep.c_pad && v0 < ep.v_pad) {
        const float* src = stg + slot * kStgLd + c * EPC;
        T tmp[EPC];
#pragma unroll
        for (int u = 0; u < EPC; ++u) tmp[u] = (T)src[u];
        *reinterpret_cast<uint4*>(G + (long long)n * ep.v_pad + v0) =
            *reinterpret_cast<const uint4*>(tmp);
      }
    }
    // G^T rows: 256 vocab x (2 segments of 32 tokens), EPC tokens per store.
    constexpr int kSegChunks = 32 / EPC;
#pragma unroll
    for (int it = 0; it < BM * 2 * kSegChunks / kThreads; ++it) {
      const int q = it * kThreads + tid;
      const int vl = q & (BM - 1);
      const int rest = q / BM;
      const int seg = rest / kSegChunks, cq = rest % kSegChunks;
      const int v = ti.tm * BM + vl;
      const int n0 = ti.tn * BN + seg * 128 + round * 32 + cq * EPC;
      if (v < ep.v_pad && n0 < ep.c_pad) {
        T tmp[EPC];
#pragma unroll
        for (int u = 0; u < EPC; ++u) tmp[u] = (T)stg[(seg * 32 + cq * EPC + u) * kStgLd + vl];
        *reinterpret_cast<uint4*>(GT + (long long)v * ep.c_pad + n0) =
            *reinterpret_cast<const uint4*>(tmp);
      }
    }
  }
}

// ------------------------------------------------------------------ dH, dW
// Plain tiles: D[m][n] (n contiguous in the output).  kAccumulate: out += D.
template <typename T, bool kAccumulate>
__global__ __launch_bounds__(kThreads, 1) void plain_gemm_kernel(Operand A, Operand B, int k_elems,
                                                                  int tiles_m, int tiles_n,
                                                                  int splits, int kb_per_split,
                                                                  float* out, long long ld_out,
                                                                  long long split_stride, int M,
                                                                  int N) {
  constexpr int BN = TILE_D, NBJ = BN / 64;
  __shared__ __attribute__((aligned(16))) char smem[Smem<BN>::kBytes];
  const TileIdx ti = map_tile<8>(tiles_m, tiles_n, splits);
  const int kb_total = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  const int kb0 = ti.split * kb_per_split;
  const int kb1 = min(kb0 + kb_per_split, kb_total);
  f32x16 acc[4][NBJ];
  gemm_mainloop<T, BN>(A, B, k_elems, ti.tm, ti.tn, kb0, kb1, smem, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, r32 = lane & 31, h = lane >> 5;
  float* o = out + ti.split * split_stride;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj) {
      const int n = ti.tn * BN + wc * (BN / 2) + bj * 32 + r32;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = ti.tm * BM + wr * 128 + bi * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) {
          float* dst = o + (long long)m * ld_out + n;
          if (kAccumulate)
            *dst += acc[bi][bj][e];
          else
            *dst = acc[bi][bj][e];
        }
      }
    }
}

template <typename T>
Operand make_operand(const void* base, long long ld_elems, int rows) {
  Operand o;
  o.base = static_cast<const char*>(base);
  o.ld = ld_elems * (long long)sizeof(T);
  o.rows = rows;
  return o;
}

template <typename T>
void fwd_impl(const void* W, int V, const void* Hc, int rows, int d, const FwdEpilogue& ep,
              hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (rows + 255) / 256;
  fwd_gemm_kernel<T><<<tiles_m * tiles_n, kThreads, 0, s>>>(
      make_operand<T>(W, d, V), make_operand<T>(Hc, d, rows), d, tiles_m, tiles_n, ep);
}

template <typename T>
void recompute_impl(const void* W, int V, const void* Hc, int rows, int d,
                    const RecomputeEpilogue& ep, hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (rows + 255) / 256;
  recompute_gemm_kernel<T><<<tiles_m * tiles_n, kThreads, 0, s>>>(
      make_operand<T>(W, d, V), make_operand<T>(Hc, d, rows), d, tiles_m, tiles_n, ep);
}

}  // namespace

void launch_fwd_gemm(DType t, const void* W, int V, const void* Hc, int rows, int d,
                     const FwdEpilogue& ep, hipStream_t s) {
  if (t == DType::BF16)
    fwd_impl<__bf16>(W, V, Hc, rows, d, ep, s);
  else
    fwd_impl<float>(W, V, Hc, rows, d, ep, s);
}

void launch_recompute_gemm(DType t, const void* W, int V, const void* Hc, int rows, int d,
                           const RecomputeEpilogue& ep, hipStream_t s) {
  if (t == DType::BF16)
    recompute_impl<__bf16>(W, V, Hc, rows, d, ep, s);
  else
    recompute_impl<float>(W, V, Hc, rows, d, ep, s);
}

void launch_dh_gemm(DType t, const void* G, int rows, int v_pad, const void* WT, int d, int splits,
                    float* part, long long split_stride, hipStream_t s) {
  const int tiles_m = (rows + BM - 1) / BM, tiles_n = (d + TILE_D - 1) / TILE_D;
  const int bk = t == DType::BF16 ? Traits<__bf16>::BK : Traits<float>::BK;
  const int kb_total = (v_pad + bk - 1) / bk;
  const int kb_per = (kb_total + splits - 1) / splits;
  const int grid = tiles_m * tiles_n * splits;
  if (t == DType::BF16)
    plain_gemm_kernel<__bf16, false><<<grid, kThreads, 0, s>>>(
        make_operand<__bf16>(G, v_pad, rows), make_operand<__bf16>(WT, v_pad, d), v_pad, tiles_m,
        tiles_n, splits, kb_per, part, d, split_stride, rows, d);
  else
    plain_gemm_kernel<float, false><<<grid, kThreads, 0, s>>>(
        make_operand<float>(G, v_pad, rows), make_operand<float>(WT, v_pad, d), v_pad, tiles_m,
        tiles_n, splits, kb_per, part, d, split_stride, rows, d);
}

void launch_dw_gemm(DType t, const void* GT, int V, int c_pad, const void* HT, int d, float* dW,
                    hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (d + TILE_D - 1) / TILE_D;
  const int bk = t == DType::BF16 ? Traits<__bf16>::BK : Traits<float>::BK;
  const int kb_total = (c_pad + bk - 1) / bk;
  const int grid = tiles_m * tiles_n;
  if (t == DType::BF16)
    plain_gemm_kernel<__bf16, true><<<grid, kThreads, 0, s>>>(
        make_operand<__bf16>(GT, c_pad, V), make_operand<__bf16>(HT, c_pad, d), c_pad, tiles_m,
        tiles_n, 1, kb_total, dW, d, 0, V, d);
  else
    plain_gemm_kernel<float, true><<<grid, kThreads, 0, s>>>(
        make_operand<float>(GT, c_pad, V), make_operand<float>(HT, c_pad, d), c_pad, tiles_m,
        tiles_n, 1, kb_total, dW, d, 0, V, d);
}

}  // namespace kd
