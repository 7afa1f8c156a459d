// kdloss C ABI: argument validation, the chunk / workspace planner, the
// per-chunk orchestration of the HIP kernels, and optional kernel timing.
#include "../../include/kdloss.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kd_internal.h"

namespace {

using kd::DType;

thread_local std::string g_last_error;
std::atomic<int> g_validate{0};

struct ValidateInit {
  ValidateInit() {
    const char* e = std::getenv("KDLOSS_VALIDATE");
    if (e != nullptr && e[0] == '1') g_validate = 1;
  }
} g_validate_init;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KD_OK;
}

// ------------------------------------------------------------------ timing
struct Record {
  const char* name;
  hipEvent_t a, b;
  double flops, bytes;
};
bool g_profile = false;
// Set while a call that creates no runtime objects runs (the no-allocation
// forward): its launches are not timed, since timing creates events.
thread_local bool g_no_events = false;
std::vector<Record> g_records;
struct Agg {
  std::string name;
  int64_t launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};
std::vector<Agg> g_agg;

struct Timed {
  Record r{};
  hipStream_t s;
  bool on;
  Timed(hipStream_t st, const char* name, double flops, double bytes)
      : s(st), on(g_profile && !g_no_events) {
    if (!on) return;
    r.name = name;
    r.flops = flops;
    r.bytes = bytes;
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
      on = false;
      return;
    }
    (void)hipEventRecord(r.a, s);
  }
  ~Timed() {
    if (!on) return;
    (void)hipEventRecord(r.b, s);
    g_records.push_back(r);
  }
};

void drain_records() {
  for (Record& r : g_records) {
    float ms = 0.f;
    (void)hipEventSynchronize(r.b);
    (void)hipEventElapsedTime(&ms, r.a, r.b);
    auto it = std::find_if(g_agg.begin(), g_agg.end(), [&](const Agg& a) { return a.name == r.name; });
    if (it == g_agg.end()) {
      g_agg.push_back(Agg{});
      it = g_agg.end() - 1;
      it->name = r.name;
    }
    it->launches += 1;
    it->ms += ms;
    it->flops += r.flops;
    it->bytes += r.bytes;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_records.clear();
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KD_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return KD_OK;
}

#define KD_LAUNCH(name, flops, bytes, call)          \
  do {                                               \
    {                                                \
      Timed _t(s, name, (double)(flops), (double)(bytes)); \
      call;                                          \
    }                                                \
    int _rc = check_launch(name);                    \
    if (_rc != KD_OK) return _rc;                    \
  } while (0)

// ------------------------------------------------------------------ planning
constexpr size_t kAlign = 256;
constexpr int64_t kMaxAutoChunk = 8192;
constexpr size_t kWorkspaceCap = size_t(24) << 30;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Layout {
  DType dt;
  int64_t n, d, V, K, chunk, c_pad, v_pad, n_vt, n_rb, splits, n_chunks, gt_cols, g_rows;
  // byte offsets
  size_t ctrl, p, S, E, hit_off, hits, common_end;
  size_t part, g, rowkl, fwd_end;
  size_t G, GT, WT, HT, dhpart, bwd_end;
};

// Split-K factor of dH = G W (K = V is long, the output C x d is small): the
// smallest factor >= 2 whose grid is a whole number of waves over the 256 CUs
// of an MI355X, else the factor in [2, 16] with the least idle tail; never
// fewer than 16 K blocks per split.  (Fewer splits also mean fewer fp32
// partials for the reduction.)
constexpr int kComputeUnits = 256;

int dh_splits(DType dt, int64_t c_pad, int64_t d, int64_t v_pad) {
  const int64_t tiles = ((c_pad + 255) / 256) * ((d + kd::TILE_D - 1) / kd::TILE_D);
  const int64_t bk = kd::k_block(dt);
  const int64_t kb_total = (v_pad + bk - 1) / bk;
  const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(16, kb_total / 16));
  int64_t best = 1;
  double best_eff = -1.0;
  for (int64_t s = std::min<int64_t>(2, s_max); s <= s_max; ++s) {
    const double waves = double(tiles * s) / kComputeUnits;
    const double eff = waves / std::ceil(waves);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
    if (eff > 0.999) break;
  }
  const int64_t kb_per = (kb_total + best - 1) / best;
  return (int)((kb_total + kb_per - 1) / kb_per);
}

Layout make_layout(DType dt, int64_t n, int64_t d, int64_t V, int64_t K, int64_t chunk) {
  Layout L{};
  L.dt = dt;
  L.n = n;
  L.d = d;
  L.V = V;
  L.K = K;
  L.chunk = chunk;
  L.c_pad = round_up(chunk, kd::KPAD);
  L.v_pad = round_up(V, kd::KPAD);
  L.n_vt = (V + kd::TILE_V - 1) / kd::TILE_V;
  L.n_rb = (n + kd::ROW_BLOCK - 1) / kd::ROW_BLOCK;
  L.splits = dh_splits(dt, L.c_pad, d, L.v_pad);
  L.n_chunks = (n + chunk - 1) / chunk;
  // G^T and H^T hold two chunks side by side, so dW runs once per pair of chunks.
  L.gt_cols = L.n_chunks > 1 ? 2 * L.c_pad : L.c_pad;
  const size_t es = kd::elem_size(dt);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.ctrl = take(sizeof(kd::Ctrl));
  L.p = take(size_t(n) * K * 4);
  L.S = take(size_t(n) * 4);
  L.E = take(size_t(n) * 4);
  L.hit_off = take(size_t(L.n_rb) * (L.n_vt + 1) * 4);
  L.hits = take(size_t(L.n_rb) * kd::ROW_BLOCK * K * sizeof(kd::Hit));
  L.common_end = o;
  // forward-only region
  L.part = take(size_t(L.n_vt) * chunk * 8);
  L.g = take(size_t(n) * K * 4);
  L.rowkl = take(size_t(n) * 4);
  L.fwd_end = o;
  // backward-only region (overlaps the forward-only one)
  o = L.common_end;
  // bf16: G holds the pair of chunks and dW reads it k-major (no G^T);
  // fp32: G holds one chunk and dW reads G^T.
  L.g_rows = L.dt == DType::BF16 ? L.gt_cols : L.c_pad;
  L.G = take(size_t(L.g_rows) * L.v_pad * es);
  L.GT = L.dt == DType::BF16 ? o : take(size_t(L.v_pad) * L.gt_cols * es);
  // bf16: dH reads W itself k-major (no W^T); fp32: dH reads W^T.
  L.WT = L.dt == DType::BF16 ? o : take(size_t(d) * L.v_pad * es);
  L.HT = take(size_t(d) * L.gt_cols * es);
  L.dhpart = take(size_t(L.splits) * L.c_pad * d * 4);
  L.bwd_end = o;
  return L;
}

int check_sizes(int dtype, int64_t n, int64_t d, int64_t V, int64_t K) {
  if (dtype != KD_BF16 && dtype != KD_F32) return fail(KD_E_INVAL, "dtype %d is not KD_BF16 or KD_F32", dtype);
  if (n <= 0 || d <= 0 || V <= 0 || K <= 0)
    return fail(KD_E_INVAL, "sizes must be positive (n=%lld d=%lld V=%lld K=%lld)", (long long)n,
                (long long)d, (long long)V, (long long)K);
  if (K > V) return fail(KD_E_INVAL, "K=%lld exceeds V=%lld", (long long)K, (long long)V);
  const int64_t epc = dtype == KD_BF16 ? 8 : 4;
  if (d % epc != 0)
    return fail(KD_E_INVAL, "d=%lld must be a multiple of %lld (16-byte rows)", (long long)d, (long long)epc);
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (n > lim || V > lim - 4096 || d > lim || (n + kd::ROW_BLOCK) * K > lim)
    return fail(KD_E_INVAL, "sizes exceed the 32-bit index range of the kernels");
  if ((V + kd::TILE_V - 1) / kd::TILE_V > kd::kMaxVocabTiles)
    return fail(KD_E_INVAL, "V=%lld exceeds the supported vocabulary of %lld", (long long)V,
                (long long)kd::kMaxVocabTiles * kd::TILE_V);
  return KD_OK;
}

int resolve_chunk(int64_t n, int64_t chunk, int64_t* out) {
  if (chunk > 0) {
    if (chunk >= n) {
      *out = n;
      return KD_OK;
    }
    if (chunk % kd::ROW_BLOCK != 0)
      return fail(KD_E_INVAL, "chunk=%lld must be a multiple of %d (or >= n)", (long long)chunk,
                  kd::ROW_BLOCK);
    *out = chunk;
    return KD_OK;
  }
  *out = 0;  // planner decides
  return KD_OK;
}

// Which workspace the automatic chunk must fit: both calls' (the planner
// query: one buffer can serve both), or only the forward's / backward's (the
// loss calls given chunk <= 0 plan against the buffer they are handed; loss
// and LSE do not depend on the chunk, so the two calls may choose differently).
enum class Fit { kBoth, kFwd, kBwd };

size_t fit_bytes(const Layout& L, Fit f) {
  return f == Fit::kFwd ? L.fwd_end : f == Fit::kBwd ? L.bwd_end : std::max(L.fwd_end, L.bwd_end);
}

int plan(int dtype, int64_t n, int64_t d, int64_t V, int64_t K, int64_t chunk, size_t budget_in,
         Layout* out, Fit fit = Fit::kBoth) {
  int rc = check_sizes(dtype, n, d, V, K);
  if (rc != KD_OK) return rc;
  int64_t c = 0;
  rc = resolve_chunk(n, chunk, &c);
  if (rc != KD_OK) return rc;
  const DType dt = static_cast<DType>(dtype);
  if (c > 0) {
    *out = make_layout(dt, n, d, V, K, c);
    return KD_OK;
  }
  size_t budget = budget_in;
  if (budget == 0) {
    size_t free_b = 0, total_b = 0;
    hipError_t e = hipMemGetInfo(&free_b, &total_b);
    if (e != hipSuccess) return fail(KD_E_HIP, "hipMemGetInfo: %s", hipGetErrorString(e));
    budget = free_b / 2;
  }
  budget = std::min(budget, kWorkspaceCap);
  if (n <= 256) {
    Layout L = make_layout(dt, n, d, V, K, n);
    if (fit_bytes(L, fit) > budget)
      return fail(KD_E_WORKSPACE, "workspace of %zu bytes exceeds the budget of %zu bytes",
                  fit_bytes(L, fit), budget);
    *out = L;
    return KD_OK;
  }
  const int64_t half = round_up((n + 1) / 2, 256);
  int64_t c_max = std::min<int64_t>(kMaxAutoChunk, std::max<int64_t>(256, half));
  for (int64_t cand = c_max; cand >= 256; cand -= 256) {
    const int64_t cc = std::min(cand, n);
    Layout L = make_layout(dt, n, d, V, K, cc);
    if (fit_bytes(L, fit) <= budget) {
      *out = L;
      return KD_OK;
    }
  }
  Layout L = make_layout(dt, n, d, V, K, std::min<int64_t>(256, n));
  return fail(KD_E_WORKSPACE, "no chunk size fits: the smallest plan (chunk 256) needs %zu bytes, budget %zu",
              fit_bytes(L, fit), budget);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_common(const void* H, const void* W, const int32_t* idx, const float* logp, void* ws,
                 size_t ws_bytes, size_t need) {
  if (H == nullptr || W == nullptr || idx == nullptr || logp == nullptr)
    return fail(KD_E_INVAL, "H, W, topk_idx and topk_logp must be non-null");
  if (!aligned16(H) || !aligned16(W)) return fail(KD_E_INVAL, "H and W must be 16-byte aligned");
  if (ws == nullptr || ws_bytes < need)
    return fail(KD_E_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                ws == nullptr ? " (null pointer)" : "");
  if (!aligned16(ws)) return fail(KD_E_INVAL, "workspace must be 16-byte aligned");
  return KD_OK;
}

// The temperature divides both sides' log-values, so it must be a positive
// finite number.
int check_temperature(float tau) {
  if (!(tau > 0.f) || !std::isfinite(tau))
    return fail(KD_E_INVAL, "temperature %g must be positive and finite", (double)tau);
  return KD_OK;
}

// Teacher preparation and bucketing shared by both calls.
int prepare_teacher(const Layout& L, const int32_t* idx, const float* logp, const uint8_t* mask,
                    float tau, char* ws, hipStream_t s) {
  auto* ctrl = reinterpret_cast<kd::Ctrl*>(ws + L.ctrl);
  const int n = (int)L.n, K = (int)L.K, V = (int)L.V;
  const double nk = double(L.n) * L.K;
  KD_LAUNCH("fill", 0, 0, kd::launch_fill_i32(reinterpret_cast<int*>(ctrl), 64, 0, s));
  KD_LAUNCH("teacher_bucket", 0, nk * 32 + L.n * 9.0,
            kd::launch_teacher_bucket(logp, idx, mask, n, K, V, 1.0f / tau,
                                      reinterpret_cast<float*>(ws + L.p),
                                      reinterpret_cast<float*>(ws + L.S),
                                      reinterpret_cast<float*>(ws + L.E),
                                      reinterpret_cast<int*>(ws + L.hit_off),
                                      reinterpret_cast<kd::Hit*>(ws + L.hits), ctrl, s));
  if (g_validate.load()) {
    kd::Ctrl host{};
    hipError_t e = hipMemcpyAsync(&host, ctrl, sizeof(int) * 2, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(KD_E_HIP, "validation read-back: %s", hipGetErrorString(e));
    if (host.range_error)
      return fail(KD_E_RANGE, "an unmasked row holds a teacher id >= V = %d", V);
  }
  return KD_OK;
}

// ------------------------------------------------------------------ teacher top-K cache builder
struct TopkLayout {
  DType dt;
  int64_t n, d, V, K, chunk, cap, n_vt, n_rb;
  size_t ctrl, zero_hits, part, lse, thr, cnt, cand, end;
};

TopkLayout make_topk_layout(DType dt, int64_t n, int64_t d, int64_t V, int64_t K, int64_t chunk,
                            int64_t cap) {
  TopkLayout L{};
  L.dt = dt;
  L.n = n;
  L.d = d;
  L.V = V;
  L.K = K;
  L.chunk = chunk;
  L.cap = cap;
  L.n_vt = (V + kd::TILE_V - 1) / kd::TILE_V;
  L.n_rb = (chunk + kd::ROW_BLOCK - 1) / kd::ROW_BLOCK;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.ctrl = take(sizeof(kd::Ctrl));
  // empty teacher-hit buckets for the statistics pass (zero offsets; the hit
  // array they index is never read)
  L.zero_hits = take(size_t(L.n_rb + 1) * (L.n_vt + 1) * 4);
  L.part = take(size_t(L.n_vt) * chunk * 8);
  L.lse = take(size_t(chunk) * 4);
  L.thr = take(size_t(chunk) * 4);
  L.cnt = take(size_t(chunk) * 4);
  L.cand = take(size_t(chunk) * cap * 8);
  L.end = o;
  return L;
}

int topk_plan(int dtype, int64_t n, int64_t d, int64_t V, int64_t K, int64_t chunk, int64_t cap,
              size_t budget_in, TopkLayout* out) {
  int rc = check_sizes(dtype, n, d, V, K);
  if (rc != KD_OK) return rc;
  if (K > kd::kMaxTopkK)
    return fail(KD_E_INVAL, "K=%lld exceeds the builder's maximum of %d", (long long)K, kd::kMaxTopkK);
  const int64_t n_vt = (V + kd::TILE_V - 1) / kd::TILE_V;
  if (n_vt > kd::kMaxTopkTiles)
    return fail(KD_E_INVAL, "V=%lld exceeds the builder's vocabulary of %lld", (long long)V,
                (long long)kd::kMaxTopkTiles * kd::TILE_V);
  // Fewer tiles than K: no tile threshold, every logit is a candidate.
  if (cap <= 0) cap = n_vt < K ? V : std::min<int64_t>(V, 4096);
  cap = std::min(cap, V);
  if (cap < K) return fail(KD_E_INVAL, "cap=%lld must be at least K=%lld", (long long)cap, (long long)K);
  int64_t c = 0;
  rc = resolve_chunk(n, chunk, &c);
  if (rc != KD_OK) return rc;
  const DType dt = static_cast<DType>(dtype);
  if (c > 0) {
    *out = make_topk_layout(dt, n, d, V, K, c, cap);
    return KD_OK;
  }
  size_t budget = budget_in;
  if (budget == 0) {
    size_t free_b = 0, total_b = 0;
    hipError_t e = hipMemGetInfo(&free_b, &total_b);
    if (e != hipSuccess) return fail(KD_E_HIP, "hipMemGetInfo: %s", hipGetErrorString(e));
    budget = free_b / 2;
  }
  budget = std::min(budget, kWorkspaceCap);
  if (n <= 256) {
    *out = make_topk_layout(dt, n, d, V, K, n, cap);
    if (out->end > budget)
      return fail(KD_E_WORKSPACE, "workspace of %zu bytes exceeds the budget of %zu bytes", out->end, budget);
    return KD_OK;
  }
  for (int64_t cc = std::min<int64_t>(kMaxAutoChunk, round_up(n, 256)); cc >= 256; cc -= 256) {
    TopkLayout L = make_topk_layout(dt, n, d, V, K, std::min(cc, n), cap);
    if (L.end <= budget) {
      *out = L;
      return KD_OK;
    }
  }
  TopkLayout L = make_topk_layout(dt, n, d, V, K, 256, cap);
  return fail(KD_E_WORKSPACE, "no chunk size fits: the smallest plan (chunk 256) needs %zu bytes, budget %zu",
              L.end, budget);
}

// The forward's launch sequence on a planned layout and a workspace of at
// least L.fwd_end bytes (arguments already checked).
int run_forward(const Layout& L, const void* H, const void* W, const int32_t* topk_idx,
                const float* topk_logp, const uint8_t* mask, float temperature, void* workspace,
                float* loss, float* lse, float* row_kl, float* gathered, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int rc = prepare_teacher(L, topk_idx, topk_logp, mask, temperature, ws, s);
  if (rc != KD_OK) return rc;

  const size_t es = kd::elem_size(L.dt);
  float* g = gathered != nullptr ? gathered : reinterpret_cast<float*>(ws + L.g);
  float* rk = row_kl != nullptr ? row_kl : reinterpret_cast<float*>(ws + L.rowkl);
  auto* part = reinterpret_cast<float2*>(ws + L.part);
  for (int64_t c0 = 0; c0 < L.n; c0 += L.chunk) {
    const int rows = (int)std::min<int64_t>(L.chunk, L.n - c0);
    kd::FwdEpilogue ep{};
    ep.part = part;
    ep.ld_part = (int)L.chunk;
    ep.n_vt = (int)L.n_vt;
    ep.c0 = (int)c0;
    ep.rows = rows;
    ep.V = (int)L.V;
    ep.K = (int)L.K;
    ep.hit_ld = (int)L.n_vt + 1;
    ep.hit_off = reinterpret_cast<const int*>(ws + L.hit_off);
    ep.hits = reinterpret_cast<const kd::Hit*>(ws + L.hits);
    ep.g = g;
    ep.inv_tau = 1.0f / temperature;
    const char* Hc = static_cast<const char*>(H) + c0 * L.d * es;
    const double fl = 2.0 * rows * L.d * L.V;
    const double by = double(L.V) * L.d * es + double(rows) * L.d * es + double(rows) * L.n_vt * 8;
    KD_LAUNCH("fwd_gemm", fl, by, kd::launch_fwd_gemm(L.dt, W, (int)L.V, Hc, rows, (int)L.d, ep, s));
    KD_LAUNCH("lse_kl", 0, double(rows) * (L.n_vt * 8 + L.K * 8 + 16),
              kd::launch_lse_kl(part, (int)L.chunk, (int)L.n_vt, (int)c0, rows,
                                reinterpret_cast<const float*>(ws + L.p), g,
                                reinterpret_cast<const float*>(ws + L.S),
                                reinterpret_cast<const float*>(ws + L.E), mask, (int)L.K,
                                temperature, lse, rk, s));
  }
  KD_LAUNCH("loss", 0, L.n * 4.0,
            kd::launch_loss(rk, (int)L.n, reinterpret_cast<const kd::Ctrl*>(ws + L.ctrl), loss, s));
  return ok();
}

// The backward's launch sequence on a planned layout (arguments checked): per
// chunk the logit gradient G (recomputed from H and W by the fused variant,
// formed from the forward's stored grids by the comparison variants), dH =
// G W, and dW (+)= G^T H per pair of chunks.
enum class Variant { kFused, kDense, kForwardChunked };

int run_backward(const Layout& L, Variant var, const float* grid, const void* H, const void* W,
                 const int32_t* topk_idx, const float* topk_logp, const uint8_t* mask, float temperature,
                 const float* lse, const float* grad_loss, void* dH, float* dW, int accumulate_dw,
                 void* workspace, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int rc = prepare_teacher(L, topk_idx, topk_logp, mask, temperature, ws, s);
  if (rc != KD_OK) return rc;

  const size_t es = kd::elem_size(L.dt);
  const bool w_kmajor = L.dt == DType::BF16;  // dH reads W itself
  if (!w_kmajor)
    KD_LAUNCH("transpose_w", 0, 2.0 * L.V * L.d * es,
              kd::launch_transpose_pad(L.dt, W, (int)L.V, (int)L.d, L.d, ws + L.WT, (int)L.v_pad,
                                       L.v_pad, s));
  bool dw_written = accumulate_dw != 0;  // later dW launches accumulate
  int pair_rows = 0;                      // unpadded rows of the pair's chunks
  for (int64_t c = 0; c < L.n_chunks; ++c) {
    const int64_t c0 = c * L.chunk;
    const int rows = (int)std::min<int64_t>(L.chunk, L.n - c0);
    const int c_pad = (int)round_up(rows, kd::KPAD);
    const int col0 = (int)((c % 2) * L.c_pad);  // this chunk's columns in G^T and H^T
    const char* Hc = static_cast<const char*>(H) + c0 * L.d * es;
    KD_LAUNCH("transpose_h", 0, 2.0 * rows * L.d * es,
              kd::launch_transpose_pad(L.dt, Hc, rows, (int)L.d, L.d, ws + L.HT + col0 * es, c_pad,
                                       L.gt_cols, s));
    const bool kmajor = L.dt == DType::BF16;  // dW reads G itself
    const int g_row0 = kmajor ? col0 : 0;
    kd::RecomputeEpilogue ep{};
    ep.G = ws + L.G;
    ep.GT = kmajor ? nullptr : ws + L.GT;
    ep.g_row0 = g_row0;
    ep.gt_ld = (int)L.gt_cols;
    ep.gt_col0 = col0;
    ep.v_pad = (int)L.v_pad;
    ep.c_pad = c_pad;
    ep.c0 = (int)c0;
    ep.rows = rows;
    ep.V = (int)L.V;
    ep.K = (int)L.K;
    ep.hit_ld = (int)L.n_vt + 1;
    ep.hit_off = reinterpret_cast<const int*>(ws + L.hit_off);
    ep.hits = reinterpret_cast<const kd::Hit*>(ws + L.hits);
    ep.S = reinterpret_cast<const float*>(ws + L.S);
    ep.lse = lse;
    ep.mask = mask;
    ep.ctrl = reinterpret_cast<const kd::Ctrl*>(ws + L.ctrl);
    ep.grad_loss = grad_loss;
    ep.tau = temperature;
    ep.inv_tau = 1.0f / temperature;
    const double fl = 2.0 * rows * L.d * L.V;
    if (var == Variant::kFused) {
      KD_LAUNCH("recompute_gemm", fl,
                double(L.V) * L.d * es + double(rows) * L.d * es + 2.0 * c_pad * L.v_pad * es,
                kd::launch_recompute_gemm(L.dt, W, (int)L.V, Hc, rows, (int)L.d, ep, s));
    } else {
      // G of this chunk from the grids the forward kept (dense: log q and the
      // teacher grid; forward-chunked: the logits and the LSE)
      const long long ldz = L.v_pad;
      const float* Zc = grid + c0 * ldz;
      const float* Pc = var == Variant::kDense ? grid + L.n * ldz + c0 * ldz : nullptr;
      KD_LAUNCH(var == Variant::kDense ? "dense_grad" : "fc_grad", 0,
                double(rows) * L.V * 4 * (var == Variant::kDense ? 2 : 1) + 2.0 * c_pad * L.v_pad * es,
                kd::launch_grad_from_grid(var == Variant::kDense, Zc, Pc, ldz, (int)L.V, (int)L.v_pad, rows,
                                          c_pad, (int)c0, lse, ep.S, mask, ep.ctrl, grad_loss, topk_idx,
                                          reinterpret_cast<const float*>(ws + L.p), (int)L.K,
                                          ws + L.G + size_t(g_row0) * L.v_pad * es, s));
    }
    const long long split_stride = (long long)L.c_pad * L.d;
    const size_t dhpart_bytes = L.bwd_end - L.dhpart;
    if (const char* why = kd::dh_launch_error(L.dt, rows, (int)L.v_pad, (int)L.d, (int)L.splits,
                                              split_stride, dhpart_bytes))
      return fail(KD_E_INVAL, "dH launch refused (%d splits, %d rows): %s", (int)L.splits, rows, why);
    bool launched = false;
    KD_LAUNCH("dh_gemm", fl,
              double(c_pad) * L.v_pad * es + double(L.d) * L.v_pad * es + double(L.splits) * rows * L.d * 4,
              launched = kd::launch_dh_gemm(L.dt, ws + L.G + size_t(g_row0) * L.v_pad * es, rows,
                                            (int)L.v_pad, w_kmajor ? W : ws + L.WT, w_kmajor, (int)L.V,
                                            (int)L.d, (int)L.splits, reinterpret_cast<float*>(ws + L.dhpart),
                                            split_stride, dhpart_bytes, s));
    if (!launched) return fail(KD_E_INVAL, "dH launch refused by its bounds check");
    KD_LAUNCH("dh_reduce", 0, double(L.splits) * rows * L.d * 4 + double(rows) * L.d * es,
              kd::launch_dh_reduce(L.dt, reinterpret_cast<const float*>(ws + L.dhpart),
                                   (int)L.splits, split_stride, rows, (int)L.d,
                                   static_cast<char*>(dH) + c0 * L.d * es, s));
    pair_rows += rows;
    if (c % 2 == 1 || c == L.n_chunks - 1) {
      const int k_len = col0 + c_pad;
      KD_LAUNCH("dw_gemm", 2.0 * pair_rows * L.d * L.V,
                double(L.V) * k_len * es + double(L.d) * k_len * es +
                    (dw_written ? 2.0 : 1.0) * L.V * L.d * 4,
                kmajor ? kd::launch_dw_gemm_kmajor(ws + L.G, (int)L.V, (int)L.v_pad, k_len, L.v_pad,
                                                   ws + L.HT, (int)L.d, L.gt_cols, dW, dw_written, s)
                       : kd::launch_dw_gemm(L.dt, ws + L.GT, (int)L.V, k_len, L.gt_cols, ws + L.HT,
                                            (int)L.d, L.gt_cols, dW, dw_written, s));
      dw_written = true;
      pair_rows = 0;
    }
  }
  return ok();
}


// ------------------------------------------------------------------ comparison variants
// The two other ways the pages compute the same loss, kept to measure the
// fused variant against on this GPU (aib.vote summary, paragraph comparing
// Dense KL, Forward-chunked KL and Fused chunked KL): dense KL builds the
// student's full log-probability grid and the teacher's full probability
// grid; forward-chunked KL computes the loss chunk by chunk with a sparse
// teacher but computes and keeps the student's full logit grid for the
// backward.  Both keep n x V fp32 grids in a caller buffer (pitch v_pad).
size_t grid_bytes_of(Variant var, int64_t n, int64_t V) {
  const size_t one = size_t(n) * size_t(round_up(V, kd::KPAD)) * 4;
  return var == Variant::kDense ? 2 * one : one;
}

int check_grid(Variant var, const void* grid, size_t grid_bytes, int64_t n, int64_t V) {
  const size_t need = grid_bytes_of(var, n, V);
  if (grid == nullptr || grid_bytes < need)
    return fail(KD_E_WORKSPACE, "grid buffer of %zu bytes needed, %zu given%s", need, grid_bytes,
                grid == nullptr ? " (null pointer)" : "");
  if (!aligned16(grid)) return fail(KD_E_INVAL, "the grid buffer must be 16-byte aligned");
  return KD_OK;
}

int comparator_fwd(Variant var, int dtype, const void* H, const void* W, const int32_t* topk_idx,
                   const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d, int64_t V, int32_t K,
                   int64_t chunk, void* grid, size_t grid_bytes, void* workspace, size_t workspace_bytes,
                   float* loss, float* lse, float* row_kl, void* stream) {
  if (dtype != KD_BF16) return fail(KD_E_INVAL, "the comparison variants take bf16 H and W only");
  Layout L;
  int rc = plan(dtype, n, d, V, K, chunk, workspace_bytes ? workspace_bytes : 1, &L, Fit::kFwd);
  if (rc != KD_OK) return rc;
  if (loss == nullptr || lse == nullptr) return fail(KD_E_INVAL, "loss and lse must be non-null");
  rc = check_common(H, W, topk_idx, topk_logp, workspace, workspace_bytes, L.fwd_end);
  if (rc != KD_OK) return rc;
  rc = check_grid(var, grid, grid_bytes, n, V);
  if (rc != KD_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  rc = prepare_teacher(L, topk_idx, topk_logp, mask, 1.0f, ws, s);
  if (rc != KD_OK) return rc;
  float* rk = row_kl != nullptr ? row_kl : reinterpret_cast<float*>(ws + L.rowkl);
  const float* p = reinterpret_cast<const float*>(ws + L.p);
  const long long ldz = L.v_pad;
  const size_t es = kd::elem_size(L.dt);
  float* Z = static_cast<float*>(grid);
  const double grid_row = double(L.V) * 4;
  if (var == Variant::kDense) {
    // the whole grids at once, as the dense loss builds them
    float* P = Z + L.n * ldz;
    KD_LAUNCH("dense_logits_gemm", 2.0 * L.n * L.d * L.V,
              double(L.V) * L.d * es + double(L.n) * L.d * es + L.n * grid_row,
              kd::launch_logits_gemm(L.dt, W, (int)L.V, H, (int)L.n, (int)L.d, Z, ldz, s));
    KD_LAUNCH("dense_log_softmax", 0, 3.0 * L.n * grid_row,
              kd::launch_log_softmax(Z, ldz, (int)L.V, (int)L.n, 0, lse, s));
    KD_LAUNCH("dense_teacher_grid", 0, L.n * grid_row + double(L.n) * L.K * 8,
              kd::launch_teacher_grid(P, ldz, (int)L.V, (int)L.n, 0, topk_idx, p, mask, (int)L.K, s));
    KD_LAUNCH("dense_kl", 0, 2.0 * L.n * grid_row,
              kd::launch_dense_kl(P, Z, ldz, (int)L.V, (int)L.n, 0, mask, rk, s));
  } else {
    float* g = reinterpret_cast<float*>(ws + L.g);
    auto* part = reinterpret_cast<float2*>(ws + L.part);
    for (int64_t c0 = 0; c0 < L.n; c0 += L.chunk) {
      const int rows = (int)std::min<int64_t>(L.chunk, L.n - c0);
      float* Zc = Z + c0 * ldz;
      const char* Hc = static_cast<const char*>(H) + c0 * L.d * es;
      KD_LAUNCH("fc_logits_gemm", 2.0 * rows * L.d * L.V,
                double(L.V) * L.d * es + double(rows) * L.d * es + rows * grid_row,
                kd::launch_logits_gemm(L.dt, W, (int)L.V, Hc, rows, (int)L.d, Zc, ldz, s));
      KD_LAUNCH("fc_row_stats", 0, rows * grid_row,
                kd::launch_row_stats(Zc, ldz, (int)L.V, rows, part, s));
      KD_LAUNCH("fc_gather", 0, double(rows) * L.K * 12,
                kd::launch_gather(Zc, ldz, rows, (int)c0, topk_idx, mask, (int)L.K, (int)L.V, g, s));
      // one (max, sum-exp) "tile" per row
      KD_LAUNCH("lse_kl", 0, double(rows) * (8 + L.K * 8 + 16),
                kd::launch_lse_kl(part, (int)L.chunk, 1, (int)c0, rows, p, g,
                                  reinterpret_cast<const float*>(ws + L.S),
                                  reinterpret_cast<const float*>(ws + L.E), mask, (int)L.K, 1.0f, lse, rk,
                                  s));
    }
  }
  KD_LAUNCH("loss", 0, L.n * 4.0,
            kd::launch_loss(rk, (int)L.n, reinterpret_cast<const kd::Ctrl*>(ws + L.ctrl), loss, s));
  return ok();
}

int comparator_bwd(Variant var, int dtype, const void* H, const void* W, const int32_t* topk_idx,
                   const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d, int64_t V, int32_t K,
                   int64_t chunk, const void* grid, size_t grid_bytes, const float* lse,
                   const float* grad_loss, void* dH, float* dW, int accumulate_dw, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (dtype != KD_BF16) return fail(KD_E_INVAL, "the comparison variants take bf16 H and W only");
  Layout L;
  int rc = plan(dtype, n, d, V, K, chunk, workspace_bytes ? workspace_bytes : 1, &L, Fit::kBwd);
  if (rc != KD_OK) return rc;
  if (lse == nullptr || grad_loss == nullptr || dH == nullptr || dW == nullptr)
    return fail(KD_E_INVAL, "lse, grad_loss, dH and dW must be non-null");
  if (!aligned16(dH) || !aligned16(dW)) return fail(KD_E_INVAL, "dH and dW must be 16-byte aligned");
  rc = check_common(H, W, topk_idx, topk_logp, workspace, workspace_bytes, L.bwd_end);
  if (rc != KD_OK) return rc;
  rc = check_grid(var, grid, grid_bytes, n, V);
  if (rc != KD_OK) return rc;
  return run_backward(L, var, static_cast<const float*>(grid), H, W, topk_idx, topk_logp, mask, 1.0f, lse,
                      grad_loss, dH, dW, accumulate_dw, workspace, stream);
}

// ------------------------------------------------------------------ no-allocation forward
// The workspace of kd_fused_chunked_kl_fwd_noalloc: a file-scope device array,
// one per GPU the library runs on, held until the process ends.  Host code
// never uses the array's name as an address (on the host it names a stand-in,
// not device memory): the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) unsigned char scratch[KD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KD_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KD_E_INVAL, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(KD_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KD_OK;
}

struct NoEvents {
  NoEvents() { g_no_events = true; }
  ~NoEvents() { g_no_events = false; }
};

}  // namespace

extern "C" {

const char* kd_status_string(int status) {
  switch (status) {
    case KD_OK: return "KD_OK";
    case KD_E_INVAL: return "KD_E_INVAL";
    case KD_E_WORKSPACE: return "KD_E_WORKSPACE";
    case KD_E_HIP: return "KD_E_HIP";
    case KD_E_RANGE: return "KD_E_RANGE";
    default: return "KD_UNKNOWN";
  }
}

const char* kd_last_error_message(void) { return g_last_error.c_str(); }

int kd_set_validate(int on) {
  g_validate = on ? 1 : 0;
  return ok();
}

int kd_profile_enable(int on) {
  g_profile = on != 0;
  return ok();
}

int kd_profile_reset(void) {
  drain_records();
  g_agg.clear();
  return ok();
}

int kd_profile_read(kd_kernel_stat_t* out, int max_entries) {
  drain_records();
  if (out == nullptr) return (int)g_agg.size();
  int m = std::min<int>(max_entries, (int)g_agg.size());
  for (int i = 0; i < m; ++i) {
    std::memset(&out[i], 0, sizeof(out[i]));
    std::snprintf(out[i].name, sizeof(out[i].name), "%s", g_agg[i].name.c_str());
    out[i].launches = g_agg[i].launches;
    out[i].total_ms = g_agg[i].ms;
    out[i].flops = g_agg[i].flops;
    out[i].bytes = g_agg[i].bytes;
  }
  return m;
}

int kd_plan_query(int dtype, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk,
                  size_t hbm_budget, kd_plan_t* out) {
  if (out == nullptr) return fail(KD_E_INVAL, "out must be non-null");
  Layout L;
  int rc = plan(dtype, n, d, V, K, chunk, hbm_budget, &L);
  if (rc != KD_OK) return rc;
  out->chunk = L.chunk;
  out->n_chunks = (L.n + L.chunk - 1) / L.chunk;
  out->vocab_tiles = L.n_vt;
  out->dh_splits = L.splits;
  out->fwd_workspace_bytes = L.fwd_end;
  out->bwd_workspace_bytes = L.bwd_end;
  out->workspace_bytes = std::max(L.fwd_end, L.bwd_end);
  return ok();
}

int kd_fused_chunked_kl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                            const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d,
                            int64_t V, int32_t K, int64_t chunk, float temperature,
                            void* workspace, size_t workspace_bytes, float* loss, float* lse,
                            float* row_kl, float* gathered, void* stream) {
  Layout L;
  // chunk <= 0: the largest automatic chunk whose forward workspace fits the
  // buffer given (an undersized buffer reports what the smallest plan needs)
  int rc = plan(dtype, n, d, V, K, chunk, workspace_bytes ? workspace_bytes : 1, &L, Fit::kFwd);
  if (rc != KD_OK) return rc;
  if (loss == nullptr || lse == nullptr) return fail(KD_E_INVAL, "loss and lse must be non-null");
  rc = check_temperature(temperature);
  if (rc != KD_OK) return rc;
  rc = check_common(H, W, topk_idx, topk_logp, workspace, workspace_bytes, L.fwd_end);
  if (rc != KD_OK) return rc;
  return run_forward(L, H, W, topk_idx, topk_logp, mask, temperature, workspace, loss, lse, row_kl,
                     gathered, stream);
}

int kd_fused_chunked_kl_fwd_noalloc(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                                    const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d,
                                    int64_t V, int32_t K, int64_t chunk, float temperature, float* loss,
                                    float* lse, float* row_kl, float* gathered, void* stream) {
  Layout L;
  int rc = plan(dtype, n, d, V, K, chunk, KD_NOALLOC_SCRATCH_BYTES, &L, Fit::kFwd);
  if (rc == KD_E_WORKSPACE)
    return fail(KD_E_WORKSPACE, "too large for the no-allocation forward's scratch of %llu bytes (%s)",
                (unsigned long long)KD_NOALLOC_SCRATCH_BYTES, g_last_error.c_str());
  if (rc != KD_OK) return rc;
  if (L.fwd_end > KD_NOALLOC_SCRATCH_BYTES)
    return fail(KD_E_WORKSPACE,
                "chunk %lld needs %zu bytes of workspace; the no-allocation forward's scratch holds %llu",
                (long long)L.chunk, L.fwd_end, (unsigned long long)KD_NOALLOC_SCRATCH_BYTES);
  if (loss == nullptr || lse == nullptr) return fail(KD_E_INVAL, "loss and lse must be non-null");
  rc = check_temperature(temperature);
  if (rc != KD_OK) return rc;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != KD_OK) return rc;
  rc = check_common(H, W, topk_idx, topk_logp, ws, KD_NOALLOC_SCRATCH_BYTES, L.fwd_end);
  if (rc != KD_OK) return rc;
  NoEvents no_events;
  return run_forward(L, H, W, topk_idx, topk_logp, mask, temperature, ws, loss, lse, row_kl, gathered,
                     stream);
}

int kd_fused_chunked_kl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                            const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d,
                            int64_t V, int32_t K, int64_t chunk, float temperature,
                            const float* lse, const float* grad_loss, void* dH, float* dW,
                            int accumulate_dw,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Layout L;
  int rc = plan(dtype, n, d, V, K, chunk, workspace_bytes ? workspace_bytes : 1, &L, Fit::kBwd);
  if (rc != KD_OK) return rc;
  if (lse == nullptr || grad_loss == nullptr || dH == nullptr || dW == nullptr)
    return fail(KD_E_INVAL, "lse, grad_loss, dH and dW must be non-null");
  if (!aligned16(dH) || !aligned16(dW)) return fail(KD_E_INVAL, "dH and dW must be 16-byte aligned");
  rc = check_temperature(temperature);
  if (rc != KD_OK) return rc;
  rc = check_common(H, W, topk_idx, topk_logp, workspace, workspace_bytes, L.bwd_end);
  if (rc != KD_OK) return rc;
  return run_backward(L, Variant::kFused, nullptr, H, W, topk_idx, topk_logp, mask, temperature, lse,
                      grad_loss, dH, dW, accumulate_dw, workspace, stream);
}

size_t kd_comparator_grid_bytes(int variant, int64_t n, int64_t V) {
  if (n <= 0 || V <= 0) return 0;
  if (variant == KD_VARIANT_DENSE) return grid_bytes_of(Variant::kDense, n, V);
  if (variant == KD_VARIANT_FORWARD_CHUNKED) return grid_bytes_of(Variant::kForwardChunked, n, V);
  return 0;
}

int kd_dense_kl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logp,
                    const uint8_t* mask, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk, void* grid,
                    size_t grid_bytes, void* workspace, size_t workspace_bytes, float* loss, float* lse,
                    float* row_kl, void* stream) {
  return comparator_fwd(Variant::kDense, dtype, H, W, topk_idx, topk_logp, mask, n, d, V, K, chunk, grid,
                        grid_bytes, workspace, workspace_bytes, loss, lse, row_kl, stream);
}

int kd_dense_kl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logp,
                    const uint8_t* mask, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk,
                    const void* grid, size_t grid_bytes, const float* lse, const float* grad_loss, void* dH,
                    float* dW, int accumulate_dw, void* workspace, size_t workspace_bytes, void* stream) {
  return comparator_bwd(Variant::kDense, dtype, H, W, topk_idx, topk_logp, mask, n, d, V, K, chunk, grid,
                        grid_bytes, lse, grad_loss, dH, dW, accumulate_dw, workspace, workspace_bytes, stream);
}

int kd_forward_chunked_kl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                              const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d, int64_t V,
                              int32_t K, int64_t chunk, void* grid, size_t grid_bytes, void* workspace,
                              size_t workspace_bytes, float* loss, float* lse, float* row_kl, void* stream) {
  return comparator_fwd(Variant::kForwardChunked, dtype, H, W, topk_idx, topk_logp, mask, n, d, V, K, chunk,
                        grid, grid_bytes, workspace, workspace_bytes, loss, lse, row_kl, stream);
}

int kd_forward_chunked_kl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                              const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d, int64_t V,
                              int32_t K, int64_t chunk, const void* grid, size_t grid_bytes, const float* lse,
                              const float* grad_loss, void* dH, float* dW, int accumulate_dw, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return comparator_bwd(Variant::kForwardChunked, dtype, H, W, topk_idx, topk_logp, mask, n, d, V, K, chunk,
                        grid, grid_bytes, lse, grad_loss, dH, dW, accumulate_dw, workspace, workspace_bytes,
                        stream);
}

int kd_teacher_topk_plan(int dtype, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk,
                         int64_t cap, size_t hbm_budget, kd_topk_plan_t* out) {
  if (out == nullptr) return fail(KD_E_INVAL, "out must be non-null");
  TopkLayout L;
  int rc = topk_plan(dtype, n, d, V, K, chunk, cap, hbm_budget, &L);
  if (rc != KD_OK) return rc;
  out->chunk = L.chunk;
  out->n_chunks = (L.n + L.chunk - 1) / L.chunk;
  out->cap = L.cap;
  out->vocab_tiles = L.n_vt;
  out->workspace_bytes = L.end;
  return ok();
}

int kd_teacher_topk(int dtype, const void* Ht, const void* Wt, int64_t n, int64_t d, int64_t V,
                    int32_t K, int64_t chunk, int64_t cap, void* workspace, size_t workspace_bytes,
                    int32_t* topk_idx, float* topk_logp, void* stream) {
  TopkLayout L;
  int rc = topk_plan(dtype, n, d, V, K, chunk, cap, workspace_bytes ? workspace_bytes : 1, &L);
  if (rc != KD_OK) return rc;
  if (Ht == nullptr || Wt == nullptr || topk_idx == nullptr || topk_logp == nullptr)
    return fail(KD_E_INVAL, "Ht, Wt, topk_idx and topk_logp must be non-null");
  if (!aligned16(Ht) || !aligned16(Wt)) return fail(KD_E_INVAL, "Ht and Wt must be 16-byte aligned");
  if (workspace == nullptr || workspace_bytes < L.end)
    return fail(KD_E_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", L.end, workspace_bytes,
                workspace == nullptr ? " (null pointer)" : "");
  if (!aligned16(workspace)) return fail(KD_E_INVAL, "workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto* ctrl = reinterpret_cast<kd::Ctrl*>(ws + L.ctrl);
  auto* zero_hits = reinterpret_cast<int*>(ws + L.zero_hits);
  auto* part = reinterpret_cast<float2*>(ws + L.part);
  auto* lse = reinterpret_cast<float*>(ws + L.lse);
  auto* thr = reinterpret_cast<float*>(ws + L.thr);
  auto* cnt = reinterpret_cast<int*>(ws + L.cnt);
  auto* cand = reinterpret_cast<int2*>(ws + L.cand);
  const size_t es = kd::elem_size(L.dt);
  KD_LAUNCH("fill", 0, 0, kd::launch_fill_i32(reinterpret_cast<int*>(ctrl), 64, 0, s));
  KD_LAUNCH("fill", 0, 0,
            kd::launch_fill_i32(zero_hits, (long long)(L.n_rb + 1) * (L.n_vt + 1), 0, s));
  for (int64_t c0 = 0; c0 < L.n; c0 += L.chunk) {
    const int rows = (int)std::min<int64_t>(L.chunk, L.n - c0);
    const char* Hc = static_cast<const char*>(Ht) + c0 * L.d * es;
    const double fl = 2.0 * rows * L.d * L.V;
    const double by = double(L.V) * L.d * es + double(rows) * L.d * es;
    kd::FwdEpilogue ep{};
    ep.part = part;
    ep.ld_part = (int)L.chunk;
    ep.n_vt = (int)L.n_vt;
    ep.c0 = 0;  // bucket keys are chunk-local here; every bucket is empty
    ep.rows = rows;
    ep.V = (int)L.V;
    ep.K = (int)L.K;
    ep.hit_ld = (int)L.n_vt + 1;
    ep.hit_off = zero_hits;
    ep.hits = reinterpret_cast<const kd::Hit*>(zero_hits);
    ep.g = nullptr;
    ep.inv_tau = 1.0f;
    KD_LAUNCH("topk_stats_gemm", fl, by + double(rows) * L.n_vt * 8,
              kd::launch_fwd_gemm(L.dt, Wt, (int)L.V, Hc, rows, (int)L.d, ep, s));
    KD_LAUNCH("topk_threshold", 0, double(rows) * (L.n_vt * 8 + 8),
              kd::launch_topk_threshold(part, (int)L.chunk, (int)L.n_vt, (int)L.K, rows, lse, thr, s));
    KD_LAUNCH("fill", 0, 0, kd::launch_fill_i32(cnt, rows, 0, s));
    kd::CandEpilogue ce{thr, cnt, cand, (int)L.cap, (int)L.V, rows};
    KD_LAUNCH("topk_cand_gemm", fl, by, kd::launch_topk_cand_gemm(L.dt, Wt, (int)L.V, Hc, rows, (int)L.d, ce, s));
    KD_LAUNCH("topk_select", 0, double(rows) * L.K * 8,
              kd::launch_topk_select(cand, (int)L.cap, cnt, lse, (int)L.K, rows, (int)c0, topk_idx,
                                     topk_logp, ctrl, s));
  }
  // An offline step: wait once, at the end, to report rows whose candidate
  // list overflowed (their entries are then incomplete).
  kd::Ctrl host{};
  hipError_t e = hipMemcpyAsync(&host, ctrl, sizeof(int) * 3, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(KD_E_HIP, "overflow read-back: %s", hipGetErrorString(e));
  if (host.overflow_rows > 0)
    return fail(KD_E_RANGE,
                "%d rows have more than cap=%lld logits at or above their top-K threshold "
                "(near-constant rows); their entries are incomplete: raise cap",
                host.overflow_rows, (long long)L.cap);
  return ok();
}

}  // extern "C"
