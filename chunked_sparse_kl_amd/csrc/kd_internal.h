// Internal declarations shared by the kdloss HIP sources: tile constants,
// the device control block and the host-side kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kd {

// Fused GEMM tiling.  The vocabulary tile (TILE_V) and the row-block size
// (ROW_BLOCK) also key the teacher-hit buckets, so every kernel that touches
// those buckets must agree on them.
constexpr int TILE_V = 256;     // vocabulary rows per fused-GEMM tile
constexpr int TILE_T = 256;     // token columns per fused-GEMM tile
constexpr int TILE_D = 256;     // hidden-dim columns per dH / dW tile
constexpr int ROW_BLOCK = 64;   // chunk starts are multiples of this many rows
constexpr int KPAD = 64;        // contraction lengths of dH / dW are padded to this
constexpr int KBLOCK_BYTES = 128;  // bytes of K per staged GEMM row (64 bf16 / 32 fp32)

// Written by the teacher-preparation kernel, read by later kernels.
struct Ctrl {
  int n_valid;       // number of unmasked rows
  int range_error;   // 1 if an unmasked row had an id outside [0, V)
  int overflow_rows; // top-K builder: rows with more candidates than their list holds
  int pad[61];
};

enum class DType { BF16 = 0, F32 = 1 };

// One unmasked teacher entry (row, k), bucketed by (vocabulary tile, 64-row
// block): its row, k, vocabulary id and the probability its scatter
// subtracts: p_{row,k}, or for an id the row repeats, the sum of the p of all
// its occurrences at the first one (in k order) and 0 at the others (the
// workspace's p array holds the same values).
struct alignas(16) Hit {
  int row;
  int k;
  int v;
  float p;
};

inline size_t elem_size(DType t) { return t == DType::BF16 ? 2 : 4; }
// K elements per GEMM main-loop block; KPAD is a multiple of it for both types.
inline int k_block(DType t) { return KBLOCK_BYTES / (int)elem_size(t); }
static_assert(KPAD % (KBLOCK_BYTES / 2) == 0, "dH / dW contractions must hold whole K blocks");

// ---------------------------------------------------------------- small kernels
void launch_fill_i32(int* p, long long count, int value, hipStream_t s);
// Teacher preparation and bucketing, one workgroup per 64-row block.  Bucket
// (row block rb, vocabulary tile j) holds the unmasked entries of rb whose id
// lies in tile j, at hits[hit_off[rb * (n_vt + 1) + j] .. hit_off[... + j + 1]);
// row block rb owns the hit range [rb * 64 * K, (rb + 1) * 64 * K).
constexpr int kMaxVocabTiles = 13307;  // LDS of one workgroup: bucket counters and repeated-id tables (64 KB)
void launch_teacher_bucket(const float* logp, const int* idx, const uint8_t* mask, int n, int K,
                           int V, float inv_tau, float* p, float* S, float* E, int* hit_off,
                           Hit* hits, Ctrl* ctrl, hipStream_t s);
void launch_lse_kl(const float2* part, int ld_part, int n_vt, int c0, int rows, const float* p,
                   const float* g, const float* S, const float* E, const uint8_t* mask, int K,
                   float tau, float* lse, float* row_kl, hipStream_t s);
void launch_loss(const float* row_kl, int n, const Ctrl* ctrl, float* loss, hipStream_t s);
void launch_transpose_pad(DType t, const void* in, int rows, int cols, long long ld_in, void* out,
                          int rows_pad, long long ld_out, hipStream_t s);
void launch_dh_reduce(DType t, const float* part, int splits, long long split_stride, int rows,
                      int d, void* dH, hipStream_t s);

// ---------------------------------------------------------------- GEMMs
struct FwdEpilogue {
  float2* part;        // [n_vt][ld_part] (max, sum-exp) per vocab tile and chunk row
  int ld_part;
  int n_vt;
  int c0;              // global row of the chunk start
  int rows;            // rows in this chunk
  int V;
  int K;
  int hit_ld;          // n_vt + 1: bucket offsets per row block
  const int* hit_off;  // [n_rb][n_vt + 1]
  const Hit* hits;     // bucketed by (row block, vocab tile)
  float* g;            // [n, K] gathered logits
  float inv_tau;       // 1 / temperature: the statistics are over z / tau
};

struct RecomputeEpilogue {
  void* G;             // [*][v_pad] dtype; this chunk's rows start at g_row0
  void* GT;            // fp32 only: [v_pad][gt_ld]; this chunk's columns start at gt_col0 (bf16: unused)
  int g_row0;
  int gt_ld;
  int gt_col0;
  int v_pad;
  int c_pad;
  int c0;
  int rows;
  int V;
  int K;
  int hit_ld;
  const int* hit_off;
  const Hit* hits;
  const float* S;      // [n]
  const float* lse;    // [n]
  const uint8_t* mask; // [n] or null
  const Ctrl* ctrl;
  const float* grad_loss;
  float tau;           // temperature: q = softmax(z / tau), G carries a factor tau
  float inv_tau;
};

// Z = W * H_c^T over one chunk (vocab rows x chunk tokens), epilogue: per
// (token, vocab tile) max / sum-exp partials and the gather at teacher ids.
void launch_fwd_gemm(DType t, const void* W, int V, const void* Hc, int rows, int d,
                     const FwdEpilogue& ep, hipStream_t s);
// Same contraction, epilogue: G = grad * w_t (S_t q - scatter p) into G and G^T.
void launch_recompute_gemm(DType t, const void* W, int V, const void* Hc, int rows, int d,
                           const RecomputeEpilogue& ep, hipStream_t s);
// part[split][c_pad][d] = G[:, split range] * W[split range, :]  (fp32 partials).
// w_kmajor (bf16 only): Wop is W itself, [V][d], read k-major through
// transposing LDS reads; otherwise Wop is W^T, [d][v_pad] (rows V .. v_pad zero).
// The launch is refused (false, nothing launched) unless dh_launch_error
// finds it in bounds for a partials buffer of part_bytes.
bool launch_dh_gemm(DType t, const void* G, int rows, int v_pad, const void* Wop, bool w_kmajor, int V,
                    int d, int splits, float* part, long long split_stride, size_t part_bytes,
                    hipStream_t s);
// nullptr if a dH launch stays inside its contraction and its partials
// buffer: 1 <= splits, every split holds at least one K block of the v_pad
// contraction, one split's partial (rows x d fp32) fits in split_stride
// floats, and splits * split_stride floats fit in part_bytes; else the reason.
const char* dh_launch_error(DType t, int rows, int v_pad, int d, int splits, long long split_stride,
                            size_t part_bytes);
// dW[V][d] (+)= G^T * H over k_len token columns (G^T rows of pitch ld_gt,
// H^T rows of pitch ld_ht); accumulate == false overwrites dW.
void launch_dw_gemm(DType t, const void* GT, int V, int k_len, long long ld_gt, const void* HT, int d,
                    long long ld_ht, float* dW, bool accumulate, hipStream_t s);
// Same from G itself ([k_len][v_pad] bf16, k-major A; k_len a multiple of 64):
// dW[V][d] (+)= G^T * H.
void launch_dw_gemm_kmajor(const void* G, int V, int v_pad, int k_len, long long ld_g, const void* HT,
                           int d, long long ld_ht, float* dW, bool accumulate, hipStream_t s);

// ---------------------------------------------------------------- comparison variants (dense, forward-chunked)
// Z[t][v] = logits of rows [0, rows) of Hc in fp32 (row pitch ldz floats, a
// multiple of 4; 16-byte aligned Z).
void launch_logits_gemm(DType t, const void* W, int V, const void* Hc, int rows, int d, float* Z,
                        long long ldz, hipStream_t s);
// part[r] = (max, sum-exp) of logit row r.
void launch_row_stats(const float* Z, long long ldz, int V, int rows, float2* part, hipStream_t s);
// In place: row r -> z - LSE(z); lse[c0 + r] = LSE(z).
void launch_log_softmax(float* Z, long long ldz, int V, int rows, int c0, float* lse, hipStream_t s);
// Dense teacher grid rows: p at the rows' ids, 0 elsewhere.
void launch_teacher_grid(float* P, long long ldz, int V, int rows, int c0, const int* idx, const float* p,
                         const uint8_t* mask, int K, hipStream_t s);
// row_kl[c0 + r] = sum_v P (log P - log q).
void launch_dense_kl(const float* P, const float* LQ, long long ldz, int V, int rows, int c0, const uint8_t* mask,
                     float* row_kl, hipStream_t s);
// g[c0 + r][k] = Z[r][i_{c0+r,k}].
void launch_gather(const float* Z, long long ldz, int rows, int c0, const int* idx, const uint8_t* mask, int K,
                   int V, float* g, hipStream_t s);
// bf16 G rows [0, c_pad) (pitch v_pad) of one chunk from stored grids: dense
// (Z = log q, P = teacher grid) or forward-chunked (Z = logits, lse).
void launch_grad_from_grid(bool dense, const float* Z, const float* P, long long ldz, int V, int v_pad, int rows,
                           int c_pad, int c0, const float* lse, const float* S, const uint8_t* mask,
                           const Ctrl* ctrl, const float* grad_loss, const int* idx, const float* p, int K,
                           void* G, hipStream_t s);

// ---------------------------------------------------------------- teacher top-K cache builder
struct CandEpilogue {
  const float* thr;    // [rows] threshold of each chunk row
  int* cnt;            // [rows] candidates seen (may exceed cap)
  int2* cand;          // [rows][cap] (id, logit bits)
  int cap;
  int V;
  int rows;
};
// Z = Wt * Ht_c^T over one chunk; every logit >= thr of its row is appended
// to that row's candidate list (the GEMM is the forward one, bit for bit).
void launch_topk_cand_gemm(DType t, const void* Wt, int V, const void* Hc, int rows, int d,
                           const CandEpilogue& ep, hipStream_t s);
// Per chunk row: LSE from the (max, sum-exp) partials, thr = the K-th largest
// tile maximum (-inf when there are fewer than K tiles).  n_vt <= kMaxTopkTiles.
constexpr int kMaxTopkTiles = 15360;  // LDS of the threshold kernel (60 KB of tile keys)
void launch_topk_threshold(const float2* part, int ld_part, int n_vt, int K, int rows, float* lse,
                           float* thr, hipStream_t s);
// Per chunk row: the K candidates with the largest logits (ties by smaller
// id), in decreasing order, as ids and logit - LSE at rows c0 + r of the
// outputs; rows whose count exceeds cap are counted in ctrl->overflow_rows.
constexpr int kMaxTopkK = 4096;  // LDS of the final sort (32 KB of keys)
void launch_topk_select(const int2* cand, int cap, const int* cnt, const float* lse, int K, int rows,
                        int c0, int* out_idx, float* out_logp, Ctrl* ctrl, hipStream_t s);

}  // namespace kd
