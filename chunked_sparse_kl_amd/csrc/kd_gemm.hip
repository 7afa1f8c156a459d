// MFMA GEMM core of kdloss (gfx950) and its four epilogues.
//
// Every contraction of the path is written as  D[m][n] = sum_k A[m][k] * B[n][k]
// with the operands K-contiguous ("NT") or, for bf16, read k-major through
// transposing LDS reads, so one main loop serves all:
//   forward / recompute:  A = W [V][d],      B = H_c [C][d]     (D = logits^T)
//   dH:                   A = G [C][V],      B = W [V][d] k-major (bf16) or
//                                            W^T [d][V] (fp32)  (split over V)
//   dW:                   A = G [2C][V] k-major (bf16) or G^T [V][2C] (fp32),
//                         B = H_c^T [d][2C]                     (pairs of chunks)
// A 512-thread workgroup (8 wavefronts in a 2 x 4 grid, two per SIMD) owns a
// 256 x 256 tile; each wavefront owns 128 x 64 and accumulates it in 32x32
// MFMA blocks (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2f32 for
// fp32).  The K loop stages 128 bytes of K per row of A and B (one K block)
// through LDS with direct-to-LDS loads into three A and two B slots: A is
// loaded two blocks ahead and B one block ahead of the block multiplied.
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

// v_max3_f32: IEEE maxNum of three values in one instruction (fmaxf would add
// canonicalising moves around each operand).
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

constexpr int BM = 256;
constexpr int ROWB = KBLOCK_BYTES;  // bytes per staged row of A or B (one K block)

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
static_assert(Traits<__bf16>::BK * 2 == ROWB && Traits<float>::BK * 4 == ROWB, "K block is one staged row");

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource of a raw (stride 0) buffer of num_records bytes at base.
__device__ inline i32x4 make_rsrc(const void* base, unsigned num_records) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = 0x00020000;
  return r;
}

__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p);
}

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.  The
// instruction has no register destination; m0, voff and the resource are read
// at issue.  The compiler does not see the LDS write, so the caller orders it
// with explicit vmcnt waits and barriers (only these loads are in flight in
// the K loop).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(i32x4 rsrc, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "m0");
}
#pragma clang diagnostic pop

// LDS of one GEMM workgroup: three K-block slots of A (BM rows) and two of B
// (BN rows), 128-byte rows; the epilogues reuse it after the K loop.
template <int BN>
struct Smem {
  static constexpr int kA = BM * ROWB;               // one A slot
  static constexpr int kB = BN * ROWB;               // one B slot
  static constexpr int kBytes = 3 * kA + 2 * kB;
  static_assert(kBytes <= 160 * 1024, "LDS of one CU");
};

#define KD_DECLARE_LDS(BN) __shared__ __attribute__((aligned(16))) char lds[Smem<BN>::kBytes]

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

// Two walks that share tiles across XCDs instead (through the last-level
// cache), measured faster for the plain GEMMs:
//  * linear: tile lin = blockIdx, so consecutive tiles run on different XCDs
//    (dW: every XCD reads the same rows of G at about the same time);
//  * M-sliced (tiles_m % 8 == 0, else the XCD ranges above): XCD x owns the
//    M tiles [x * tiles_m / 8, ...) and all XCDs walk the N tiles (then the
//    splits) in step (dH: every XCD reads the same W tiles).
template <int kGroupM>
__device__ inline TileIdx map_tile_linear(int tiles_m, int tiles_n, int splits) {
  const int lin = blockIdx.x;
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

template <int kGroupM>
__device__ inline TileIdx map_tile_msliced(int tiles_m, int tiles_n, int splits) {
  if ((tiles_m & 7) != 0) return map_tile<kGroupM>(tiles_m, tiles_n, splits);
  const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
  const int mpx = tiles_m >> 3;
  const int per = mpx * tiles_n;
  TileIdx t;
  t.split = l / per;
  const int r = l - t.split * per;
  t.tm = xcd * mpx + r % mpx;
  t.tn = r / mpx;
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
  int krows;          // k-major B only: k rows present in memory (later ones read as zero)
};

// Main loop: accumulates the tile (tm, tn) over K blocks [kb0, kb1).
//
// Operands move global -> LDS by direct-to-LDS buffer loads
// (buffer_load_dwordx4 ... lds): one wavefront instruction writes 8 staged
// rows of 128 bytes (1 KB) at a wave-uniform LDS address, lane L at +16 L, so
// the 8 lanes of a row fetch one whole 128-byte line (half-line rows double
// the L1 -> L2 request count, which then limits the loop).  The XOR swizzle of
// the 16-byte chunks is applied on the global side: lane L fetches chunk
// (L%8) ^ ((row/2)%8) of its row, so LDS holds chunk c of row r at position
// c ^ ((r/2)%8) and a fragment read by 16 consecutive rows touches 16 distinct
// 16-byte bank groups (64 banks).  Each tile gets a buffer resource covering
// exactly its valid rows; lanes of rows past the operand end use an
// out-of-range offset (skipped by the hardware range check; those rows'
// results are never stored).  The one K block that runs past the contraction
// end is loaded through registers with ordinary buffer loads, whose
// out-of-range chunks read as zero.
// kAT: A is stored k-major ([k][m], m contiguous; bf16 only).  Its K block is
// then 64 staged rows of BM elements (512 bytes): one load instruction fills
// two such rows, 16-byte chunk c of row k sits at c ^ 4 (k % 4), and the MFMA
// fragments come from transposing LDS reads (ds_read_b64_tr_b16).  The block's
// buffer resource is rebased per K block, so the operand may exceed 4 GB.
// kBT: the same for B ([k][n], n contiguous; bf16 only), whose K extent may
// end inside the last K block (its range then stops at the last k row).
template <typename T, int BN, int WC, bool kAT = false, bool kBT = false>
struct MainLoop {
  static_assert(!kAT || sizeof(T) == 2, "k-major A needs 16-bit elements");
  static_assert(!kBT || (sizeof(T) == 2 && !kAT), "k-major B: 16-bit elements, A k-contiguous");
  static constexpr int BK = Traits<T>::BK;
  static constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  static constexpr int WAVES = 2 * WC;            // 2 wavefront rows x WC columns
  static constexpr int ROWS_PER_LD = 8 * WAVES;   // staged rows written by one instruction index
  static constexpr int KROWS_PER_LD = 2 * WAVES;  // k-major: k rows (of BM / BN elements) per instruction index
  static constexpr int A_LD = BM / ROWS_PER_LD;   // per-wavefront load instructions per K block (A)
  static constexpr int B_LD = BN / ROWS_PER_LD;
  static constexpr int LOADS = A_LD + B_LD;
  static constexpr int NBJ = BN / (32 * WC);      // 32-column MFMA blocks per wavefront
  static constexpr int SUB = ROWB / 32;           // MFMA substeps (32 bytes of K) per block
  static constexpr unsigned kOut = 0x80000000u;   // beyond any tile's num_records

  i32x4 ra, rb;
  const char* a_tile;        // first row of the tile (for the ragged block's ordinary loads)
  const char* b_tile;
  unsigned a_bytes, b_bytes; // bytes of the tile's valid rows
  unsigned a_off, b_off;     // this lane's byte offset for load i = 0 (row r, chunk c)
  unsigned a_step, b_step;   // ROWS_PER_LD rows, bytes
  int a_valid, b_valid;      // valid rows of the tile
  int r;                     // this lane's row within its wavefront's 8
  int c;                     // logical chunk fetched by this lane
  int k_elems;
  int wave_row;              // wave * 8 (uniform)
  long long a_ld;            // kAT: bytes per k row of A
  long long b_ldk;           // kBT: bytes per k row of B
  int b_krows;               // kBT: k rows of B in memory

  __device__ inline void init(const Operand& A, const Operand& B, int ke, int tm, int tn) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wave_row = w * 8;
    r = lane >> 3;
    c = (lane & 7) ^ (((wave_row + r) >> 1) & 7);
    k_elems = ke;
    if constexpr (kAT) {
      // A.rows is the m extent; lane L of load i stages k row 2 WAVES i + 2 w + L / 32,
      // physical chunk L % 32, i.e. logical chunk (L % 32) ^ 4 (row % 4).
      const int row = 2 * w + (lane >> 5);
      const int ca = (lane & 31) ^ (4 * (row & 3));
      a_valid = min(A.rows - tm * BM, BM);
      a_tile = A.base + (long long)tm * BM * (long long)sizeof(T);
      a_ld = A.ld;
      a_off = (ca * EPC < a_valid) ? (unsigned)(row * A.ld + ca * 16) : kOut;
      a_step = (unsigned)(KROWS_PER_LD * A.ld);
      b_valid = min(B.rows - tn * BN, BN);
      b_tile = B.base + (long long)tn * BN * B.ld;
      b_bytes = (unsigned)(b_valid * B.ld);
      rb = make_rsrc(b_tile, b_bytes);
      b_off = (unsigned)((wave_row + r) * B.ld + c * 16);
      b_step = (unsigned)(ROWS_PER_LD * B.ld);
      return;
    }
    a_valid = min(A.rows - tm * BM, BM);
    b_valid = min(B.rows - tn * BN, BN);
    a_tile = A.base + (long long)tm * BM * A.ld;
    a_bytes = (unsigned)(a_valid * A.ld);
    ra = make_rsrc(a_tile, a_bytes);
    a_off = (unsigned)((wave_row + r) * A.ld + c * 16);
    a_step = (unsigned)(ROWS_PER_LD * A.ld);
    if constexpr (kBT) {
      // as k-major A: lane L of load i stages k row 2 WAVES i + 2 w + L / 32 of
      // the block, logical chunk (L % 32) ^ 4 (row % 4) of its BN columns
      static_assert(BN == BM && B_LD == A_LD, "k-major B staging mirrors k-major A");
      const int row = 2 * w + (lane >> 5);
      const int cb = (lane & 31) ^ (4 * (row & 3));
      b_tile = B.base + (long long)tn * BN * (long long)sizeof(T);
      b_ldk = B.ld;
      b_krows = B.krows;
      b_off = (cb * EPC < b_valid) ? (unsigned)(row * B.ld + cb * 16) : kOut;
      b_step = (unsigned)(KROWS_PER_LD * B.ld);
      return;
    }
    b_tile = B.base + (long long)tn * BN * B.ld;
    b_bytes = (unsigned)(b_valid * B.ld);
    rb = make_rsrc(b_tile, b_bytes);
    b_off = (unsigned)((wave_row + r) * B.ld + c * 16);
    b_step = (unsigned)(ROWS_PER_LD * B.ld);
  }

  // Load instruction i of the full K block kb into the A slot `st` (i < A_LD)
  // or the B slot (i < B_LD).  With valid == false every lane is out of
  // range: the instruction still counts in vmcnt (so every step waits for the
  // same count) but reads nothing.
  __device__ inline void issue_a(int kb, char* st, bool valid, int i) const {
    if constexpr (kAT) {
      const i32x4 rk = make_rsrc(a_tile + (long long)kb * BK * a_ld, (unsigned)(BK * a_ld));
      const unsigned off = (valid && a_off != kOut) ? a_off + i * a_step : kOut;
      dma16(rk, off, __builtin_amdgcn_readfirstlane(lds_addr(st + (KROWS_PER_LD * i + wave_row / 4) * BM * (int)sizeof(T))));
      return;
    }
    const unsigned off = (valid && wave_row + r + ROWS_PER_LD * i < a_valid) ? a_off + i * a_step + (unsigned)kb * ROWB : kOut;
    dma16(ra, off, __builtin_amdgcn_readfirstlane(lds_addr(st + (i * ROWS_PER_LD + wave_row) * ROWB)));
  }
  __device__ inline void issue_b(int kb, char* st, bool valid, int i) const {
    if constexpr (kBT) {
      const int k0 = kb * BK;
      const int rows_here = max(0, min(BK, b_krows - k0));  // k rows of this block in memory
      const i32x4 rk = make_rsrc(b_tile + (long long)k0 * b_ldk, (unsigned)(rows_here * b_ldk));
      const unsigned off = (valid && b_off != kOut) ? b_off + i * b_step : kOut;
      dma16(rk, off, __builtin_amdgcn_readfirstlane(lds_addr(st + (KROWS_PER_LD * i + wave_row / 4) * BN * (int)sizeof(T))));
      return;
    }
    const unsigned off = (valid && wave_row + r + ROWS_PER_LD * i < b_valid) ? b_off + i * b_step + (unsigned)kb * ROWB : kOut;
    dma16(rb, off, __builtin_amdgcn_readfirstlane(lds_addr(st + (i * ROWS_PER_LD + wave_row) * ROWB)));
  }
  __device__ inline void issue_all_a(int kb, char* st, bool valid) const {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) issue_a(kb, st, valid, i);
  }
  __device__ inline void issue_all_b(int kb, char* st, bool valid) const {
#pragma unroll
    for (int i = 0; i < B_LD; ++i) issue_b(kb, st, valid, i);
  }

  // The K block that runs past the contraction end, through registers: chunks
  // at k >= k_elems read as zero (out-of-range offset of an ordinary load).
  __device__ inline void load_ragged(int kb, char* sa, char* sb) const {
    const unsigned koff = (unsigned)kb * ROWB;
    const bool k_ok = kb * BK + c * EPC < k_elems;
    const int lane_pos = (threadIdx.x & 63) * 16;
    const __amdgpu_buffer_rsrc_t ba =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a_tile), (short)0, (int)a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t bb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b_tile), (short)0, (int)b_bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const unsigned off = (k_ok && wave_row + r + ROWS_PER_LD * i < a_valid) ? a_off + i * a_step + koff : kOut;
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ba, off, 0, 0));
      *reinterpret_cast<uint4*>(sa + (i * ROWS_PER_LD + wave_row) * ROWB + lane_pos) = v;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const unsigned off = (k_ok && wave_row + r + ROWS_PER_LD * i < b_valid) ? b_off + i * b_step + koff : kOut;
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bb, off, 0, 0));
      *reinterpret_cast<uint4*>(sb + (i * ROWS_PER_LD + wave_row) * ROWB + lane_pos) = v;
    }
  }

  struct Frags {
    uint4 a[4], b[NBJ];
  };

  // Fragments of NBLK 32-wide blocks, starting at column idx0, of a k-major
  // slot (rows of row_bytes per k).  Lane l of 16-lane group g names k row
  // kb + (l%16)/4 and columns idx0 + 16 (g%2) + 4 (l % 4) .. +3; the
  // transposing read hands lane i of the group the 4 k values of column
  // ... + i.  Two reads give k = 16 s + 8 h .. +7.  k % 4 = (l % 16) / 4 for
  // every read, so the swizzle term depends on the lane and the block only
  // and the rest is an immediate offset.
  template <int NBLK, int kRowBytes>
  __device__ inline static void tr_frags(const char* slot, int idx0, int s, uint4 (&out)[NBLK]) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, q = lane & 15, x = q >> 2;
    const int m = idx0 + 16 * (g & 1) + 4 * (q & 3);
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) char lds_char;
    lds_char* const base = (lds_char*)const_cast<char*>(slot) + ((8 * (g >> 1) + x) * kRowBytes + (m & 7) * 2);
#pragma unroll
    for (int bi = 0; bi < NBLK; ++bi) {
      lds_char* const a = base + ((((m >> 3) + 4 * bi) ^ (4 * x)) << 4);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(a + (16 * s) * kRowBytes));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(a + (16 * s + 4) * kRowBytes));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      out[bi] = uint4{l2.x, l2.y, h2.x, h2.y};
    }
  }

  // Fragment loads of substep s (16 bf16 / 8 fp32 K elements) from the slots
  // sa (A) and sb (B).
  __device__ inline static void load(const char* sa, const char* sb, int s, Frags& f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave / WC, wc = wave % WC;
    const int r32 = lane & 31, h = lane >> 5;
    const int ch = ((2 * s + h) ^ ((r32 >> 1) & 7)) << 4;
    if constexpr (kBT) {
      tr_frags<NBJ, BN * 2>(sb, wc * (BN / WC), s, f.b);
    } else {
      const char* b_row0 = sb + (wc * (BN / WC) + r32) * ROWB;
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj) f.b[bj] = *reinterpret_cast<const uint4*>(b_row0 + bj * 32 * ROWB + ch);
    }
    if constexpr (kAT) {
      tr_frags<4, BM * 2>(sa, wr * 128, s, f.a);
    } else {
      const char* a_row0 = sa + (wr * 128 + r32) * ROWB;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) f.a[bi] = *reinterpret_cast<const uint4*>(a_row0 + bi * 32 * ROWB + ch);
    }
  }

  __device__ inline static void mma(const Frags& f, f32x16 (&acc)[4][NBJ]) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj) mma_block<T>(f.a[bi], f.b[bj], acc[bi][bj]);
  }

  // One substep: MFMAs on `cur` while the fragments of the next substep are
  // read into `nxt` (one LDS read after each MFMA).
  __device__ inline static void substep(const char* sa, const char* sb, int s_next, const Frags& cur,
                                        Frags& nxt, f32x16 (&acc)[4][NBJ]) {
    load(sa, sb, s_next, nxt);
    mma(cur, acc);
#pragma unroll
    for (int g = 0; g < 4 + NBJ; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// s_waitcnt vmcnt(n) lgkmcnt(0).
template <int N>
__device__ inline void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}

// K-block slots: block j's A lives in A slot j % 3, its B in B slot j % 2.
// A is loaded two blocks ahead and B one block ahead, so about one and a half
// blocks are in flight while one is multiplied.
template <int BN>
struct Slots {
  char* lds;
  __device__ inline char* a(int i) const { return lds + i * Smem<BN>::kA; }
  __device__ inline char* b(int i) const { return lds + 3 * Smem<BN>::kA + i * Smem<BN>::kB; }
};

template <typename T, int BN, int WC, bool kAT = false, bool kBT = false>
struct KLoop {
  using ML = MainLoop<T, BN, WC, kAT, kBT>;
  ML ml;
  Slots<BN> sl;
  int kb_full;
  typename ML::Frags fa;  // substep-0 fragments of the block about to be multiplied

  // Multiplies K block j (slot phase t = j - kb0 mod 6, fa: its substep-0
  // fragments).  Substeps 0..2 each read the next substep's fragments.
  // Before the last substep every wavefront waits until its loads of block
  // j+1 have landed (only A of j+2 may still be in flight) and its own LDS
  // reads are done; the barrier (without a memory fence, which would wait for
  // everything) then publishes j+1 and frees block j's slots.  The last
  // substep's MFMAs overlap the substep-0 reads of j+1 and the loads of B of
  // j+2 and A of j+3 into the freed slots.
  template <int t>
  __device__ inline void step(int j, f32x16 (&acc)[4][ML::NBJ]) {
    static_assert(ML::SUB == 4, "four substeps per K block");
    char* const ca = sl.a(t % 3);
    char* const cb = sl.b(t % 2);
    typename ML::Frags fb;
    ML::substep(ca, cb, 1, fa, fb, acc);
    ML::substep(ca, cb, 2, fb, fa, acc);
    ML::substep(ca, cb, 3, fa, fb, acc);
    wait_vmcnt_lgkm0<ML::A_LD>();
    __builtin_amdgcn_s_barrier();
    const bool vb = j + 2 < kb_full, va = j + 3 < kb_full;
    ML::load(sl.a((t + 1) % 3), sl.b((t + 1) % 2), 0, fa);
    int q = 0;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < ML::NBJ; ++bj) {
        mma_block<T>(fb.a[bi], fb.b[bj], acc[bi][bj]);
        // one load per MFMA block: B of j+2 first, then A of j+3
        if (q < ML::B_LD) ml.issue_b(j + 2, cb, vb, q);
        else if (q < ML::LOADS) ml.issue_a(j + 3, ca, va, q - ML::B_LD);
        ++q;
      }
#pragma unroll
    for (; q < ML::LOADS; ++q) {
      if (q < ML::B_LD) ml.issue_b(j + 2, cb, vb, q);
      else ml.issue_a(j + 3, ca, va, q - ML::B_LD);
    }
#pragma unroll
    for (int g = 0; g < 4 + ML::NBJ; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// Forced inline: several kernels instantiate the same main loop and epilogue,
// and an out-of-line call would pass the accumulators through scratch memory.
template <typename T, int BN, int WC, bool kAT = false, bool kBT = false>
__device__ __attribute__((always_inline)) inline void gemm_mainloop(const Operand& A, const Operand& B, int k_elems, int tm, int tn,
                                     int kb0, int kb1, char* lds,
                                     f32x16 (&acc)[4][BN / (32 * WC)]) {
  using ML = MainLoop<T, BN, WC, kAT, kBT>;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < ML::NBJ; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  KLoop<T, BN, WC, kAT, kBT> L;
  L.sl.lds = lds;
  L.ml.init(A, B, k_elems, tm, tn);
  L.kb_full = min(kb1, k_elems / ML::BK);  // blocks entirely inside the contraction
  const int kb_full = L.kb_full;
  // Same issue order as the steady state: ..., A(j), B(j), A(j+1), B(j+1), A(j+2).
  L.ml.issue_all_a(kb0 + 0, L.sl.a(0), kb0 + 0 < kb_full);
  L.ml.issue_all_b(kb0 + 0, L.sl.b(0), kb0 + 0 < kb_full);
  L.ml.issue_all_a(kb0 + 1, L.sl.a(1), kb0 + 1 < kb_full);
  L.ml.issue_all_b(kb0 + 1, L.sl.b(1), kb0 + 1 < kb_full);
  L.ml.issue_all_a(kb0 + 2, L.sl.a(2), kb0 + 2 < kb_full);
  wait_vmcnt<2 * ML::A_LD + ML::B_LD>();  // block kb0 landed
  __builtin_amdgcn_s_barrier();
  ML::load(L.sl.a(0), L.sl.b(0), 0, L.fa);
  int kb = kb0;
  for (; kb + 6 <= kb_full; kb += 6) {
    L.template step<0>(kb + 0, acc);
    L.template step<1>(kb + 1, acc);
    L.template step<2>(kb + 2, acc);
    L.template step<3>(kb + 3, acc);
    L.template step<4>(kb + 4, acc);
    L.template step<5>(kb + 5, acc);
  }
  if (kb + 0 < kb_full) L.template step<0>(kb + 0, acc);
  if (kb + 1 < kb_full) L.template step<1>(kb + 1, acc);
  if (kb + 2 < kb_full) L.template step<2>(kb + 2, acc);
  if (kb + 3 < kb_full) L.template step<3>(kb + 3, acc);
  if (kb + 4 < kb_full) L.template step<4>(kb + 4, acc);
  wait_vmcnt<0>();      // the trailing out-of-range loads, before LDS is reused
  __syncthreads();
  if (!kAT && !kBT && kb_full < kb1) {  // ragged last block (at most one; never k-major)
    char* const sa = L.sl.a(0);
    char* const sb = L.sl.b(0);
    L.ml.load_ragged(kb_full, sa, sb);
    __syncthreads();
    typename ML::Frags f0, f1;
    ML::load(sa, sb, 0, f0);
    ML::substep(sa, sb, 1, f0, f1, acc);
    ML::substep(sa, sb, 2, f1, f0, acc);
    ML::substep(sa, sb, 3, f0, f1, acc);
    ML::mma(f1, acc);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ fused epilogues
// The fused kernels use 8 wavefronts in a 2 x 4 grid; wavefront (wr, wc) owns
// vocabulary rows [128 wr, +128) and tokens [64 wc, +64) of the 256 x 256
// tile as 4 x 2 blocks of 32 x 32.  Its 64 tokens are exactly one 64-row block
// of the teacher-hit buckets (chunks start at multiples of 64 rows), so each
// wavefront finds the teacher entries of its tokens in one bucket and applies
// them to its own accumulators: no workgroup-wide staging, no barriers.
constexpr int kFusedWC = 4;
constexpr int kFusedThreads = 128 * kFusedWC;
constexpr int kFusedNBJ = 2;
static_assert(256 / kFusedWC == ROW_BLOCK, "a wavefront's tokens form one hit row block");

// Register q = 16 * (2 bi + bj) + e of this lane's accumulators (q uniform
// over the wavefront, so the switch is a scalar branch and the element is
// picked by register-relative addressing).
// Accumulator register q = 16 * (2 bi + bj) + e of this lane, q uniform over
// the wavefront: a switch with constant register indices, i.e. a scalar
// branch tree (a runtime index would send the accumulators to scratch).
#define KD_GET(q) \
  case q:         \
    return acc[(q) >> 5][((q) >> 4) & 1][(q) & 15];
#define KD_ADD(q)                               \
  case q:                                       \
    acc[(q) >> 5][((q) >> 4) & 1][(q) & 15] += x; \
    break;
__device__ inline float acc_get(const f32x16 (&acc)[4][kFusedNBJ], int q) {
  switch (q) {
    KD_GET(0) KD_GET(1) KD_GET(2) KD_GET(3) KD_GET(4) KD_GET(5) KD_GET(6) KD_GET(7) KD_GET(8) KD_GET(9) KD_GET(10) KD_GET(11) KD_GET(12) KD_GET(13) KD_GET(14) KD_GET(15)
    KD_GET(16) KD_GET(17) KD_GET(18) KD_GET(19) KD_GET(20) KD_GET(21) KD_GET(22) KD_GET(23) KD_GET(24) KD_GET(25) KD_GET(26) KD_GET(27) KD_GET(28) KD_GET(29) KD_GET(30) KD_GET(31)
    KD_GET(32) KD_GET(33) KD_GET(34) KD_GET(35) KD_GET(36) KD_GET(37) KD_GET(38) KD_GET(39) KD_GET(40) KD_GET(41) KD_GET(42) KD_GET(43) KD_GET(44) KD_GET(45) KD_GET(46) KD_GET(47)
    KD_GET(48) KD_GET(49) KD_GET(50) KD_GET(51) KD_GET(52) KD_GET(53) KD_GET(54) KD_GET(55) KD_GET(56) KD_GET(57) KD_GET(58) KD_GET(59) KD_GET(60) KD_GET(61) KD_GET(62) KD_GET(63)
    KD_GET(64) KD_GET(65) KD_GET(66) KD_GET(67) KD_GET(68) KD_GET(69) KD_GET(70) KD_GET(71) KD_GET(72) KD_GET(73) KD_GET(74) KD_GET(75) KD_GET(76) KD_GET(77) KD_GET(78) KD_GET(79)
    KD_GET(80) KD_GET(81) KD_GET(82) KD_GET(83) KD_GET(84) KD_GET(85) KD_GET(86) KD_GET(87) KD_GET(88) KD_GET(89) KD_GET(90) KD_GET(91) KD_GET(92) KD_GET(93) KD_GET(94) KD_GET(95)
    KD_GET(96) KD_GET(97) KD_GET(98) KD_GET(99) KD_GET(100) KD_GET(101) KD_GET(102) KD_GET(103) KD_GET(104) KD_GET(105) KD_GET(106) KD_GET(107) KD_GET(108) KD_GET(109) KD_GET(110) KD_GET(111)
    KD_GET(112) KD_GET(113) KD_GET(114) KD_GET(115) KD_GET(116) KD_GET(117) KD_GET(118) KD_GET(119) KD_GET(120) KD_GET(121) KD_GET(122) KD_GET(123) KD_GET(124) KD_GET(125) KD_GET(126) KD_GET(127)
  }
  return 0.f;
}

__device__ inline void acc_add(f32x16 (&acc)[4][kFusedNBJ], int q, float x) {
  switch (q) {
    KD_ADD(0) KD_ADD(1) KD_ADD(2) KD_ADD(3) KD_ADD(4) KD_ADD(5) KD_ADD(6) KD_ADD(7) KD_ADD(8) KD_ADD(9) KD_ADD(10) KD_ADD(11) KD_ADD(12) KD_ADD(13) KD_ADD(14) KD_ADD(15)
    KD_ADD(16) KD_ADD(17) KD_ADD(18) KD_ADD(19) KD_ADD(20) KD_ADD(21) KD_ADD(22) KD_ADD(23) KD_ADD(24) KD_ADD(25) KD_ADD(26) KD_ADD(27) KD_ADD(28) KD_ADD(29) KD_ADD(30) KD_ADD(31)
    KD_ADD(32) KD_ADD(33) KD_ADD(34) KD_ADD(35) KD_ADD(36) KD_ADD(37) KD_ADD(38) KD_ADD(39) KD_ADD(40) KD_ADD(41) KD_ADD(42) KD_ADD(43) KD_ADD(44) KD_ADD(45) KD_ADD(46) KD_ADD(47)
    KD_ADD(48) KD_ADD(49) KD_ADD(50) KD_ADD(51) KD_ADD(52) KD_ADD(53) KD_ADD(54) KD_ADD(55) KD_ADD(56) KD_ADD(57) KD_ADD(58) KD_ADD(59) KD_ADD(60) KD_ADD(61) KD_ADD(62) KD_ADD(63)
    KD_ADD(64) KD_ADD(65) KD_ADD(66) KD_ADD(67) KD_ADD(68) KD_ADD(69) KD_ADD(70) KD_ADD(71) KD_ADD(72) KD_ADD(73) KD_ADD(74) KD_ADD(75) KD_ADD(76) KD_ADD(77) KD_ADD(78) KD_ADD(79)
    KD_ADD(80) KD_ADD(81) KD_ADD(82) KD_ADD(83) KD_ADD(84) KD_ADD(85) KD_ADD(86) KD_ADD(87) KD_ADD(88) KD_ADD(89) KD_ADD(90) KD_ADD(91) KD_ADD(92) KD_ADD(93) KD_ADD(94) KD_ADD(95)
    KD_ADD(96) KD_ADD(97) KD_ADD(98) KD_ADD(99) KD_ADD(100) KD_ADD(101) KD_ADD(102) KD_ADD(103) KD_ADD(104) KD_ADD(105) KD_ADD(106) KD_ADD(107) KD_ADD(108) KD_ADD(109) KD_ADD(110) KD_ADD(111)
    KD_ADD(112) KD_ADD(113) KD_ADD(114) KD_ADD(115) KD_ADD(116) KD_ADD(117) KD_ADD(118) KD_ADD(119) KD_ADD(120) KD_ADD(121) KD_ADD(122) KD_ADD(123) KD_ADD(124) KD_ADD(125) KD_ADD(126) KD_ADD(127)
  }
}
#undef KD_GET
#undef KD_ADD

// The teacher entries of one wavefront: the bucket of (the 64-row block of its
// tokens, vocabulary tile tm).  The first 64 entries (one per lane) are
// loaded before the K loop so their latency hides under it.
struct WaveHits {
  int lo, hi;      // bucket range in the hit array
  int row0;        // global row of the wavefront's first token
  int v_lo;        // first vocabulary id of the wavefront's 128 rows
  Hit pre;         // this lane's entry among the first 64

  __device__ inline void init(const int* hit_off, const Hit* hits, int hit_ld, int tm, int c0, int rows,
                              int tok0, int v_lo_) {
    const int lane = threadIdx.x & 63;
    row0 = c0 + tok0;
    v_lo = v_lo_;
    lo = hi = 0;
    if (tok0 < rows) {  // tokens past the chunk end have no bucket
      const int key = (row0 / ROW_BLOCK) * hit_ld + tm;
      lo = hit_off[key];
      hi = hit_off[key + 1];
    }
    pre.row = pre.k = 0;
    pre.v = -1;
    pre.p = 0.f;
    if (lo + lane < hi) pre = hits[lo + lane];
  }

  // Calls f(q, owner, row, k, p) for each entry whose id falls in the
  // wavefront's vocabulary rows: accumulator register q of lane `owner`
  // holds that (token, id) logit.
  template <class F>
  __device__ inline void for_each(const Hit* hits, F&& f) const {
    const int lane = threadIdx.x & 63;
    for (int base = lo; base < hi; base += 64) {
      Hit hk = pre;
      if (base != lo) {
        hk.v = -1;
        if (base + lane < hi) hk = hits[base + lane];
      }
      const int cnt = min(64, hi - base);
      for (int u = 0; u < cnt; ++u) {
        const int vl = __builtin_amdgcn_readlane(hk.v, u) - v_lo;
        if ((unsigned)vl >= 128u) continue;
        const int row = __builtin_amdgcn_readlane(hk.row, u);
        const int k = __builtin_amdgcn_readlane(hk.k, u);
        const float p = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hk.p), u));
        const int tl = row - row0;  // 0..63
        const int r = vl & 31;
        const int q = ((((vl >> 5) << 1) | (tl >> 5)) << 4) | ((r >> 3) << 2) | (r & 3);
        const int owner = (tl & 31) | (((r >> 2) & 1) << 5);
        f(q, owner, row, k, p);
      }
    }
  }
};

// ------------------------------------------------------------------ forward
// D[v][t] = z_{t,v}.  Per token: max and sum of exp(z/tau - max) over this
// tile's vocabulary rows (-> one (max, sum) partial of the softened logits per
// vocabulary tile; tau > 0, so max(z/tau) = max(z)/tau); the raw logits at the
// token's teacher ids are read straight out of the accumulators.
template <typename T>
__global__ __launch_bounds__(kFusedThreads, 1) void fwd_gemm_kernel(Operand A, Operand B, int k_elems,
                                                                     int tiles_m, int tiles_n,
                                                                     FwdEpilogue ep) {
  constexpr int BN = 256, NBJ = kFusedNBJ, WC = kFusedWC;
  KD_DECLARE_LDS(BN);
  const TileIdx ti = map_tile<4>(tiles_m, tiles_n, 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC, r32 = lane & 31, h = lane >> 5;
  WaveHits wh;
  wh.init(ep.hit_off, ep.hits, ep.hit_ld, ti.tm, ep.c0, ep.rows, ti.tn * BN + wc * 64,
          ti.tm * BM + wr * 128);
  f32x16 acc[4][NBJ];
  const int kb_end = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  gemm_mainloop<T, BN, WC>(A, B, k_elems, ti.tm, ti.tn, 0, kb_end, lds, acc);

  // --- gather the logits at the teacher ids that fall in this wavefront's block
  wh.for_each(ep.hits, [&](int q, int owner, int row, int k, float) {
    const float z = acc_get(acc, q);
    if (lane == owner) ep.g[(long long)row * ep.K + k] = z;
  });

  // --- per-token (max, sum-exp) over this wavefront's 128 vocabulary rows.
  // Only the last vocabulary tile has rows past V: they are set to -inf once
  // (a uniform branch), so the two passes below need no per-element test.
  if ((ti.tm + 1) * BM > ep.V) {
    const int v_base = ti.tm * BM + wr * 128 + 4 * h;  // + bi*32 + 8*i + j
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (v_base + bi * 32 + 8 * (e >> 2) + (e & 3) >= ep.V) acc[bi][bj][e] = kNegInf;
  }
  float tmax[NBJ], tsum[NBJ];
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    float mx = kNegInf;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = max3f(mx, acc[bi][bj][e], acc[bi][bj][e + 1]);
    {
      // the other half-wavefront's value (lane i ^ 32) by a register swap of
      // the halves: {own, partner} for lanes 0-31, {partner, own} above
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mx),
                                                      __builtin_bit_cast(unsigned, mx), false, false);
      const unsigned r0 = r[0], r1 = r[1];  // (a bit_cast of a vector element would read element 0)
      mx = max3f(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1), mx);
    }
    float sm = 0.f;
    const float sc = kLog2e * ep.inv_tau;
    if (mx != kNegInf) {
      const float mxs = mx * sc;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e) sm += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[bi][bj][e], sc, -mxs));
    }
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, sm),
                                                      __builtin_bit_cast(unsigned, sm), false, false);
      const unsigned r0 = r[0], r1 = r[1];
      sm = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    }
    tmax[bj] = mx * ep.inv_tau;
    tsum[bj] = sm;
  }
  // --- merge the two vocabulary halves (wr = 0, 1) through LDS
  float2* red = reinterpret_cast<float2*>(lds);
  if (h == 0) {
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
      red[wr * BN + (wc * NBJ + bj) * 32 + r32] = make_float2(tmax[bj], tsum[bj]);
  }
  __syncthreads();
  if (tid < BN) {
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
}

// ------------------------------------------------------------------ recompute
// D[v][t] = z_{t,v} again; G_{t,v} = gw*S_t*q_{t,v} - gw*sum_k p_{t,k}[i_{t,k} = v]
// with q = softmax(z / tau) and gw = tau * grad_loss * mask_t / N_valid (the
// derivative of tau^2 KL through z / tau), formed in the accumulators (the
// scatter goes straight into the owning registers), rounded to T and written
// row-major (G, through a per-wavefront LDS block so the stores are whole
// rows) and, for fp32 only, transposed (G^T, straight from registers: a
// lane's 32-token column is contiguous there).
template <typename T>
__global__ __launch_bounds__(kFusedThreads, 1) void recompute_gemm_kernel(Operand A, Operand B,
                                                                           int k_elems, int tiles_m,
                                                                           int tiles_n,
                                                                           RecomputeEpilogue ep) {
  constexpr int BN = 256, NBJ = kFusedNBJ, WC = kFusedWC;
  KD_DECLARE_LDS(BN);
  const TileIdx ti = map_tile<4>(tiles_m, tiles_n, 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC, r32 = lane & 31, h = lane >> 5;
  const int n_wave = ti.tn * BN + wc * 64;  // chunk-local first token of this wavefront
  const int v_wave = ti.tm * BM + wr * 128; // first vocabulary row of this wavefront
  WaveHits wh;
  wh.init(ep.hit_off, ep.hits, ep.hit_ld, ti.tm, ep.c0, ep.rows, n_wave, v_wave);
  f32x16 acc[4][NBJ];
  const int kb_end = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  gemm_mainloop<T, BN, WC>(A, B, k_elems, ti.tm, ti.tn, 0, kb_end, lds, acc);

  const int nv = ep.ctrl->n_valid;
  const float gw = nv > 0 ? ep.tau * ep.grad_loss[0] / (float)nv : 0.f;
  const float sc = kLog2e * ep.inv_tau;
  // bf16 G: coef * 2^(z sc - lse2) with coef = gw S_t (S_t >= 0, so coef has
  // gw's sign) is formed as sign(gw) * 2^(z sc - (lse2 - log2 |coef|)): one FMA
  // and one exp per element, no multiply and no select.  Its magnitude is off
  // by a few fp32 ulps, far below the rounding to bf16.  A row without gradient
  // (masked, past the chunk end, or coef = 0) gets the offset +inf and so
  // 2^-inf = 0 everywhere.  The teacher entries below are applied to the
  // magnitude and the sign comes last.  fp32 G keeps the product form.
  constexpr bool kLogScale = sizeof(T) == 2;
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    const int n = n_wave + bj * 32 + r32;
    const int t = ep.c0 + n;
    const bool live = n < ep.rows && (ep.mask == nullptr || ep.mask[t] != 0);
    if constexpr (kLogScale) {
      const float mag = live ? fabsf(gw) * ep.S[t] : 0.f;
      const float off = mag > 0.f ? ep.lse[t] * kLog2e - __builtin_amdgcn_logf(mag) : __builtin_inff();
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc[bi][bj][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[bi][bj][e], sc, -off));
    } else {
      const float coef = live ? gw * ep.S[t] : 0.f;
      const float lse2 = live ? ep.lse[t] * kLog2e : 0.f;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[bi][bj][e], sc, -lse2));
          acc[bi][bj][e] = live ? coef * q : 0.f;
        }
    }
  }
  if ((ti.tm + 1) * BM > ep.V) {  // last vocabulary tile: rows past V carry no gradient
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (v_wave + bi * 32 + 8 * (e >> 2) + 4 * h + (e & 3) >= ep.V) acc[bi][bj][e] = 0.f;
  }
  // Teacher entries: G -= gw * p at (t, i_{t,k}) (masked rows have none);
  // bf16: |gw| p off the magnitude, then the sign of gw.
  const float gp = kLogScale ? fabsf(gw) : gw;
  wh.for_each(ep.hits, [&](int q, int owner, int, int, float p) {
    acc_add(acc, q, lane == owner ? -gp * p : 0.f);
  });
  if (kLogScale && gw < 0.f) {  // uniform: a negative incoming gradient
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[bi][bj][e] = -acc[bi][bj][e];
  }

  T* G = static_cast<T*>(ep.G);
  // --- G^T[v][n] (fp32 only: the bf16 dW GEMM reads G itself k-major): for
  // a fixed register, the 32 lanes of a half-wavefront hold 32 consecutive
  // tokens of one vocabulary row.
  if constexpr (sizeof(T) == 4) {
    T* GT = static_cast<T*>(ep.GT);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj) {
        const int n = n_wave + bj * 32 + r32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v0 = v_wave + bi * 32 + 8 * i + 4 * h;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v0 + j < ep.v_pad && n < ep.c_pad)
              __builtin_nontemporal_store((T)acc[bi][bj][4 * i + j], GT + (long long)(v0 + j) * ep.gt_ld + ep.gt_col0 + n);
        }
      }
  }
  // --- G[n][v]: each wavefront stages its 32-token x 128-row blocks (rounded
  // to T) in its own LDS rows and stores whole 128-value rows.
  constexpr int kPitch = 128 * (int)sizeof(T) + 16;    // bytes per staged token row
  constexpr int kChunks = 128 * (int)sizeof(T) / 16;   // 16-byte chunks per row
  constexpr int EPC = 16 / sizeof(T);
  static_assert(8 * 32 * kPitch <= Smem<BN>::kBytes, "per-wavefront G staging");
  char* const reg = lds + wave * 32 * kPitch;
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        T v4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = (T)acc[bi][bj][4 * i + j];
        char* dst = reg + r32 * kPitch + (bi * 32 + 8 * i + 4 * h) * (int)sizeof(T);
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(v4);
        else
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v4);
      }
#pragma unroll
    for (int it = 0; it < 32 * kChunks / 64; ++it) {
      const int q = it * 64 + lane;
      const int row = q / kChunks, c = q % kChunks;
      const uint4 val = *reinterpret_cast<const uint4*>(reg + row * kPitch + c * 16);
      const int n = n_wave + bj * 32 + row;
      const int v = v_wave + c * EPC;
      if (n < ep.c_pad && v < ep.v_pad)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, val),
                                    reinterpret_cast<u32x4*>(G + (long long)(ep.g_row0 + n) * ep.v_pad + v));
    }
  }
}

// ------------------------------------------------------------------ logits (comparators)
// D[v][t] = z_{t,v}, stored as it is: Z[t][v] in fp32 (row pitch ldz floats,
// a multiple of 4) for the comparison variants that keep the logits.  For a
// fixed register group a lane holds 4 consecutive vocabulary rows of one
// token, stored as one 16-byte vector (element by element at the V end).
template <typename T>
__global__ __launch_bounds__(kFusedThreads, 1) void logits_gemm_kernel(Operand A, Operand B, int k_elems,
                                                                        int tiles_m, int tiles_n, float* Z,
                                                                        long long ldz, int V, int rows) {
  constexpr int BN = 256, NBJ = kFusedNBJ, WC = kFusedWC;
  KD_DECLARE_LDS(BN);
  const TileIdx ti = map_tile<4>(tiles_m, tiles_n, 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC, r32 = lane & 31, h = lane >> 5;
  f32x16 acc[4][NBJ];
  const int kb_end = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  gemm_mainloop<T, BN, WC>(A, B, k_elems, ti.tm, ti.tn, 0, kb_end, lds, acc);
  const int v_wave = ti.tm * BM + wr * 128;
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    const int t = ti.tn * BN + wc * 64 + bj * 32 + r32;
    float* const zr = Z + (long long)t * ldz;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = v_wave + bi * 32 + 8 * i + 4 * h;
        if (t >= rows) continue;
        if (v + 3 < V) {
          *reinterpret_cast<f32x4*>(zr + v) = f32x4{acc[bi][bj][4 * i], acc[bi][bj][4 * i + 1],
                                                   acc[bi][bj][4 * i + 2], acc[bi][bj][4 * i + 3]};
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v + j < V) zr[v + j] = acc[bi][bj][4 * i + j];
        }
      }
  }
}

// ------------------------------------------------------------------ top-K candidates
// D[v][t] = z_{t,v}, the same main loop as the forward statistics pass, so the
// logits are bitwise those whose tile maxima set the thresholds.  Each logit
// at or above its row's threshold is appended to the row's list (an atomic
// cursor per row; a few hundred entries per row at V = 201088, K = 100).
template <typename T>
__global__ __launch_bounds__(kFusedThreads, 1) void topk_cand_gemm_kernel(Operand A, Operand B,
                                                                           int k_elems, int tiles_m,
                                                                           int tiles_n, CandEpilogue ep) {
  constexpr int BN = 256, NBJ = kFusedNBJ, WC = kFusedWC;
  KD_DECLARE_LDS(BN);
  const TileIdx ti = map_tile<4>(tiles_m, tiles_n, 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC, r32 = lane & 31, h = lane >> 5;
  f32x16 acc[4][NBJ];
  const int kb_end = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  gemm_mainloop<T, BN, WC>(A, B, k_elems, ti.tm, ti.tn, 0, kb_end, lds, acc);
  const int v_base = ti.tm * BM + wr * 128 + 4 * h;  // + bi*32 + 8*(e/4) + e%4
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    const int n = ti.tn * BN + wc * 64 + bj * 32 + r32;
    const float t = n < ep.rows ? ep.thr[n] : __builtin_inff();
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = v_base + bi * 32 + 8 * (e >> 2) + (e & 3);
        const float z = acc[bi][bj][e];
        if (z >= t && v < ep.V) {
          const int slot = atomicAdd(&ep.cnt[n], 1);
          if (slot < ep.cap) ep.cand[(long long)n * ep.cap + slot] = make_int2(v, __builtin_bit_cast(int, z));
        }
      }
  }
}

// ------------------------------------------------------------------ dH, dW
// Plain tiles: D[m][n] (n contiguous in the output).  kAccumulate: out += D.
constexpr int kPlainWC = 4;                    // wavefront columns of the dH / dW tiles
constexpr int kPlainThreads = 128 * kPlainWC;

// Tile walks of the plain GEMMs (measured per kernel).
enum class Walk { kMSliced, kLinear };

template <typename T, bool kAccumulate, Walk kWalk, bool kAT = false, bool kBT = false>
__device__ __attribute__((always_inline)) inline void plain_gemm(char* lds, Operand A, Operand B, int k_elems, int tiles_m,
                                  int tiles_n, int splits, int kb_per_split, float* out,
                                  long long ld_out, long long split_stride, int M, int N) {
  constexpr int BN = TILE_D, WC = kPlainWC, NBJ = BN / (32 * WC);
  const TileIdx ti = kWalk == Walk::kMSliced ? map_tile_msliced<8>(tiles_m, tiles_n, splits)
                                             : map_tile_linear<4>(tiles_m, tiles_n, splits);
  const int kb_total = (k_elems + Traits<T>::BK - 1) / Traits<T>::BK;
  const int kb0 = ti.split * kb_per_split;
  const int kb1 = min(kb0 + kb_per_split, kb_total);
  f32x16 acc[4][NBJ];
  gemm_mainloop<T, BN, WC, kAT, kBT>(A, B, k_elems, ti.tm, ti.tn, kb0, kb1, lds, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WC, wc = wave % WC, r32 = lane & 31, h = lane >> 5;
  float* o = out + ti.split * split_stride;
  constexpr int NB = 4 * NBJ;  // 32x32 blocks of this wavefront, b = bi * NBJ + bj
  auto row0 = [&](int b) { return ti.tm * BM + wr * 128 + (b / NBJ) * 32 + 4 * h; };
  auto col = [&](int b) { return ti.tn * BN + wc * (BN / WC) + (b % NBJ) * 32 + r32; };
  if (kAccumulate) {
    // out += D.  The old values of block b + kAhead are loaded before block b
    // is stored (in program order, since loads and stores may alias), so
    // their latency overlaps; the K loop's fragment registers are free now.
    // Buffer accesses over this tile's valid rows with an out-of-range offset
    // for elements outside the output keep the code free of branches (so the
    // compiler can count outstanding loads precisely).
    constexpr int kAhead = 3;
    const int m_tile = ti.tm * BM;
    const int rows_ok = min(M - m_tile, BM);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        o + (long long)m_tile * ld_out, (short)0, (int)(rows_ok * ld_out * 4), 0x00020000);
    // Rows past the output end fall outside num_records by themselves; a
    // column past N gets bit 31 added (arithmetic, not a select, which the
    // compiler would turn back into branches).
    auto off = [&](int b, int e) -> unsigned {
      const int n = col(b), m = row0(b) + 8 * (e >> 2) + (e & 3);
      const unsigned past = (unsigned)(N - 1 - n) >> 31;
      return (unsigned)(((m - m_tile) * ld_out + n) * 4) + (past << 31);
    };
    float old[NB][16];
    auto load = [&](int b) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        old[b][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off(b, e), 0, 0));
    };
#pragma unroll
    for (int b = 0; b < kAhead; ++b) load(b);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + kAhead < NB) load(b + kAhead);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, old[b][e] + acc[b / NBJ][b % NBJ][e]), rs,
                                              off(b, e), 0, 0);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int n = col(b), m0 = row0(b);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 8 * (e >> 2) + (e & 3);
        if (n < N && m < M) o[(long long)m * ld_out + n] = acc[b / NBJ][b % NBJ][e];
      }
    }
  }
}

// Distinct kernel names for dH (split-K partials, plain stores) and dW
// (accumulated into the caller's fp32 dW).
template <typename T, bool kBT>
__global__ __launch_bounds__(kPlainThreads, 1) void dh_gemm_kernel(Operand A, Operand B, int k_elems,
                                                                    int tiles_m, int tiles_n, int splits,
                                                                    int kb_per_split, float* out,
                                                                    long long ld_out,
                                                                    long long split_stride, int M, int N) {
  KD_DECLARE_LDS(TILE_D);
  plain_gemm<T, false, Walk::kMSliced, false, kBT>(lds, A, B, k_elems, tiles_m, tiles_n, splits,
                                                   kb_per_split, out, ld_out, split_stride, M, N);
}

template <typename T, bool kAccumulate, bool kAT>
__global__ __launch_bounds__(kPlainThreads, 1) void dw_gemm_kernel(Operand A, Operand B, int k_elems,
                                                                    int tiles_m, int tiles_n,
                                                                    int kb_per_split, float* out,
                                                                    long long ld_out, int M, int N) {
  KD_DECLARE_LDS(TILE_D);
  plain_gemm<T, kAccumulate, Walk::kLinear, kAT>(lds, A, B, k_elems, tiles_m, tiles_n, 1, kb_per_split,
                                                  out, ld_out, 0, M, N);
}

template <typename T>
Operand make_operand(const void* base, long long ld_elems, int rows) {
  Operand o;
  o.base = static_cast<const char*>(base);
  o.ld = ld_elems * (long long)sizeof(T);
  o.rows = rows;
  o.krows = 0;
  return o;
}

template <typename T>
void fwd_impl(const void* W, int V, const void* Hc, int rows, int d, const FwdEpilogue& ep,
              hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (rows + 255) / 256;
  fwd_gemm_kernel<T><<<tiles_m * tiles_n, kFusedThreads, 0, s>>>(
      make_operand<T>(W, d, V), make_operand<T>(Hc, d, rows), d, tiles_m, tiles_n, ep);
}

template <typename T>
void recompute_impl(const void* W, int V, const void* Hc, int rows, int d,
                    const RecomputeEpilogue& ep, hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (rows + 255) / 256;
  recompute_gemm_kernel<T><<<tiles_m * tiles_n, kFusedThreads, 0, s>>>(
      make_operand<T>(W, d, V), make_operand<T>(Hc, d, rows), d, tiles_m, tiles_n, ep);
}

template <typename T>
void logits_impl(const void* W, int V, const void* Hc, int rows, int d, float* Z, long long ldz,
                 hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (rows + 255) / 256;
  logits_gemm_kernel<T><<<tiles_m * tiles_n, kFusedThreads, 0, s>>>(
      make_operand<T>(W, d, V), make_operand<T>(Hc, d, rows), d, tiles_m, tiles_n, Z, ldz, V, rows);
}

template <typename T>
void topk_cand_impl(const void* Wt, int V, const void* Hc, int rows, int d, const CandEpilogue& ep,
                    hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (rows + 255) / 256;
  topk_cand_gemm_kernel<T><<<tiles_m * tiles_n, kFusedThreads, 0, s>>>(
      make_operand<T>(Wt, d, V), make_operand<T>(Hc, d, rows), d, tiles_m, tiles_n, ep);
}

}  // namespace

void launch_topk_cand_gemm(DType t, const void* Wt, int V, const void* Hc, int rows, int d,
                           const CandEpilogue& ep, hipStream_t s) {
  if (t == DType::BF16)
    topk_cand_impl<__bf16>(Wt, V, Hc, rows, d, ep, s);
  else
    topk_cand_impl<float>(Wt, V, Hc, rows, d, ep, s);
}

void launch_logits_gemm(DType t, const void* W, int V, const void* Hc, int rows, int d, float* Z,
                        long long ldz, hipStream_t s) {
  if (t == DType::BF16)
    logits_impl<__bf16>(W, V, Hc, rows, d, Z, ldz, s);
  else
    logits_impl<float>(W, V, Hc, rows, d, Z, ldz, s);
}

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

const char* dh_launch_error(DType t, int rows, int v_pad, int d, int splits, long long split_stride,
                            size_t part_bytes) {
  if (rows <= 0 || v_pad <= 0 || d <= 0) return "empty operand";
  if (splits < 1) return "splits must be at least 1";
  const long long bk = k_block(t);
  const long long kb_total = (v_pad + bk - 1) / bk;
  if (splits > kb_total) return "more splits than K blocks in the contraction";
  const long long kb_per = (kb_total + splits - 1) / splits;
  if ((splits - 1) * kb_per >= kb_total) return "a split would hold no K block";
  if ((long long)rows * d > split_stride) return "one split's partial exceeds the split stride";
  if ((unsigned long long)splits * (unsigned long long)split_stride * 4ull > part_bytes)
    return "the partials of all splits exceed the partials buffer";
  return nullptr;
}

bool launch_dh_gemm(DType t, const void* G, int rows, int v_pad, const void* Wop, bool w_kmajor, int V,
                    int d, int splits, float* part, long long split_stride, size_t part_bytes,
                    hipStream_t s) {
  if (dh_launch_error(t, rows, v_pad, d, splits, split_stride, part_bytes) != nullptr) return false;
  const int tiles_m = (rows + BM - 1) / BM, tiles_n = (d + TILE_D - 1) / TILE_D;
  const int bk = k_block(t);
  const int kb_total = (v_pad + bk - 1) / bk;
  const int kb_per = (kb_total + splits - 1) / splits;
  const int grid = tiles_m * tiles_n * splits;
  if (t == DType::BF16 && w_kmajor) {
    // B = W itself, [V][d]: k-major, n extent d, V k rows (rows V .. v_pad read as zero)
    Operand B = make_operand<__bf16>(Wop, d, d);
    B.krows = V;
    dh_gemm_kernel<__bf16, true><<<grid, kPlainThreads, 0, s>>>(
        make_operand<__bf16>(G, v_pad, rows), B, v_pad, tiles_m, tiles_n, splits, kb_per, part, d,
        split_stride, rows, d);
  } else if (t == DType::BF16) {
    dh_gemm_kernel<__bf16, false><<<grid, kPlainThreads, 0, s>>>(
        make_operand<__bf16>(G, v_pad, rows), make_operand<__bf16>(Wop, v_pad, d), v_pad, tiles_m,
        tiles_n, splits, kb_per, part, d, split_stride, rows, d);
  } else {
    dh_gemm_kernel<float, false><<<grid, kPlainThreads, 0, s>>>(
        make_operand<float>(G, v_pad, rows), make_operand<float>(Wop, v_pad, d), v_pad, tiles_m,
        tiles_n, splits, kb_per, part, d, split_stride, rows, d);
  }
  return true;
}

template <typename T, bool kAcc, bool kAT>
void dw_impl(const void* A, int V, int a_rows, int k_len, long long ld_a, const void* HT, int d,
             long long ld_ht, float* dW, hipStream_t s) {
  const int tiles_m = (V + BM - 1) / BM, tiles_n = (d + TILE_D - 1) / TILE_D;
  const int kb_total = (k_len + Traits<T>::BK - 1) / Traits<T>::BK;
  dw_gemm_kernel<T, kAcc, kAT><<<tiles_m * tiles_n, kPlainThreads, 0, s>>>(
      make_operand<T>(A, ld_a, a_rows), make_operand<T>(HT, ld_ht, d), k_len, tiles_m, tiles_n,
      kb_total, dW, d, V, d);
}

void launch_dw_gemm(DType t, const void* GT, int V, int k_len, long long ld_gt, const void* HT, int d,
                    long long ld_ht, float* dW, bool accumulate, hipStream_t s) {
  if (t == DType::BF16) {
    if (accumulate) dw_impl<__bf16, true, false>(GT, V, V, k_len, ld_gt, HT, d, ld_ht, dW, s);
    else dw_impl<__bf16, false, false>(GT, V, V, k_len, ld_gt, HT, d, ld_ht, dW, s);
  } else {
    if (accumulate) dw_impl<float, true, false>(GT, V, V, k_len, ld_gt, HT, d, ld_ht, dW, s);
    else dw_impl<float, false, false>(GT, V, V, k_len, ld_gt, HT, d, ld_ht, dW, s);
  }
}

void launch_dw_gemm_kmajor(const void* G, int V, int v_pad, int k_len, long long ld_g, const void* HT,
                           int d, long long ld_ht, float* dW, bool accumulate, hipStream_t s) {
  if (accumulate) dw_impl<__bf16, true, true>(G, V, v_pad, k_len, ld_g, HT, d, ld_ht, dW, s);
  else dw_impl<__bf16, false, true>(G, V, v_pad, k_len, ld_g, HT, d, ld_ht, dW, s);
}

}  // namespace kd
