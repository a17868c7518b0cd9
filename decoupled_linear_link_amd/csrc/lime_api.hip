// C ABI of the LIME hot path: argument validation, launch planning and the
// kernel launches.  Every check that the host can make happens before the
// first launch, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "lime.h"
#include "common.h"
#include "generic_kernels.h"
#include "mfma_kernels.h"
#include "user_kernels.h"

using namespace lime;

namespace {

thread_local std::string g_err;

lime_status_t fail(lime_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lime_status_t ok() {
  g_err.clear();
  return LIME_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// Kernel timing for measurement tools (lime_trace_begin / lime_trace_end).
// While a trace is open, each launch takes a pair of events that the
// runtime stamps with the dispatch's own start and end times
// (hipExtLaunchKernelGGL); otherwise launches are plain.
struct Trace {
  std::mutex m;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> ev;  // start, end per slot
  std::vector<const char*> name;
  int n = 0, dropped = 0;
};
Trace g_trace;

// the event pair of the next launch, or nulls when no trace is open or it is
// full
void trace_slot(const char* name, hipEvent_t* e0, hipEvent_t* e1) {
  *e0 = *e1 = nullptr;
  if (!g_trace.on.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> lk(g_trace.m);
  if (!g_trace.on.load(std::memory_order_relaxed)) return;
  if (static_cast<size_t>(g_trace.n) >= g_trace.name.size()) {
    ++g_trace.dropped;
    return;
  }
  *e0 = g_trace.ev[2 * g_trace.n];
  *e1 = g_trace.ev[2 * g_trace.n + 1];
  g_trace.name[g_trace.n++] = name;
}

// a kernel launch under a trace name (the kernel's name in the source)
#define LIME_LAUNCH(NAME, KERNEL, GRID, BLOCK, LDS, STREAM, ...)                          \
  do {                                                                                   \
    hipEvent_t e0_, e1_;                                                                 \
    trace_slot(NAME, &e0_, &e1_);                                                        \
    if (e0_ != nullptr)                                                                  \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, e0_, e1_, 0, __VA_ARGS__); \
    else                                                                                 \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                 \
  } while (0)

#define LIME_CHECK_LAUNCH(what)                                                          \
  do {                                                                                   \
    hipError_t e_ = hipGetLastError();                                                   \
    if (e_ != hipSuccess)                                                                \
      return fail(LIME_ERR_HIP, "%s: %s", what, hipGetErrorString(e_));                  \
  } while (0)

bool dh_supported(int dh) { return dh == 16 || dh == 32 || dh == 64 || dh == 128; }

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <typename K>
int blocks_per_cu_lds(K kernel, int threads, size_t lds) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, lds) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

template <typename K>
int blocks_per_cu(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

// ---------------------------------------------------------------------------
// QK cache: matrix-core kernel for the shapes it is instantiated for
// ---------------------------------------------------------------------------
template <int ELL, int D, int H, bool I8>
lime_status_t launch_qk_mfma(const void* items, const void* keys, void* cache, float* qscale,
                             int64_t n_items, float scale, int phi, hipStream_t st) {
  using C = mfma::QkCfg<ELL, D, H, I8>;
  if constexpr (!I8) {
    // bf16: item tiles by LDS-DMA, two in flight per workgroup
    using Q = mfma::QkDmaCfg<ELL, D, H>;
    auto k = mfma::qk_cache_dma<ELL, D, H>;
    constexpr size_t lds = Q::lds_bytes;
    static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(lds)) == hipSuccess;
    (void)attr;
    static const int per_cu = blocks_per_cu_lds(k, C::NT, lds);
    const int64_t ntiles = (n_items + C::TI - 1) / C::TI;
    int64_t grid = static_cast<int64_t>(cu_count()) * per_cu;
    if (grid > ntiles) grid = ntiles;
    LIME_LAUNCH("qk_cache", k, dim3(static_cast<unsigned>(grid)), dim3(C::NT), lds, st,
                       static_cast<const bf16_t*>(items), static_cast<const bf16_t*>(keys),
                       static_cast<bf16_t*>(cache), n_items, scale, phi, ntiles);
    LIME_CHECK_LAUNCH("qk cache build (mfma)");
    return ok();
  }
  auto k = mfma::qk_cache<ELL, D, H, I8>;
  static const int per_cu = blocks_per_cu(k, C::NT);
  const int64_t ntiles = (n_items + C::TI - 1) / C::TI;
  int64_t grid = static_cast<int64_t>(cu_count()) * per_cu;
  if (grid > ntiles) grid = ntiles;
  LIME_LAUNCH(I8 ? "qk_cache_i8" : "qk_cache", k, dim3(static_cast<unsigned>(grid)), dim3(C::NT), 0, st,
                     static_cast<const bf16_t*>(items), static_cast<const bf16_t*>(keys), cache, qscale,
                     n_items, scale, phi, ntiles);
  LIME_CHECK_LAUNCH("qk cache build (mfma)");
  return ok();
}

// returns LIME_ERR_UNSUPPORTED (without launching) if no instantiation fits
template <bool I8>
lime_status_t try_qk_mfma(int ell, int d, int H, const void* items, const void* keys, void* cache,
                          float* qscale, int64_t n_items, float scale, int phi, hipStream_t st) {
#define LIME_QK(E, DD, HH) \
  if (ell == E && d == DD && H == HH) return launch_qk_mfma<E, DD, HH, I8>(items, keys, cache, qscale, n_items, scale, phi, st);
  LIME_QK(32, 64, 2)
  LIME_QK(32, 128, 4)
  LIME_QK(64, 128, 4)
  LIME_QK(32, 256, 8)
  LIME_QK(64, 256, 8)
#undef LIME_QK
  return LIME_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------------------
// candidate scoring: matrix-core kernel for d_h = 32, ell in {32, 64}
// ---------------------------------------------------------------------------
template <int ELL, int H, bool I8>
lime_status_t launch_cs_mfma(const void* cache, const float* qscale, int64_t n_items, const void* lp,
                             const int64_t* ids, const int64_t* off, int B, int64_t total_M,
                             void* out, int* bad, hipStream_t st) {
  constexpr int NG = H < 4 ? 1 : H / 4;  // head groups per candidate tile (one wave each)
  const int64_t ntiles = (total_M + 15) / 16;
  // about 16 waves per CU; a short list (one tile or less per such wave)
  // gets 8 per CU, so that each wave walks two or more tiles and its
  // software-pipelined gathers overlap (65,536 candidates at ell = 64:
  // 24 -> 22 us; 1M candidates keep 16, where 8 was 11% slower)
  const int64_t wpc = ntiles <= static_cast<int64_t>(cu_count()) * 16 ? 8 : 16;
  const int64_t target_waves = static_cast<int64_t>(cu_count()) * wpc / NG;
  int64_t tpw = (ntiles + target_waves - 1) / target_waves;
  if (tpw < 1) tpw = 1;
  const int64_t waves = (ntiles + tpw - 1) / tpw * NG;
  const int64_t grid = (waves + 3) / 4;
  LIME_LAUNCH(I8 ? "cand_score_i8" : "cand_score", (mfma::cand_score<ELL, H, I8>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     cache, qscale, n_items, static_cast<const bf16_t*>(lp), ids, off, B, total_M,
                     static_cast<bf16_t*>(out), bad, tpw);
  LIME_CHECK_LAUNCH("candidate scoring (mfma)");
  return ok();
}

template <bool I8>
lime_status_t try_cs_mfma(int ell, int d, int H, const void* cache, const float* qscale, int64_t n_items,
                          const void* lp, const int64_t* ids, const int64_t* off, int B, int64_t total_M,
                          void* out, int* bad, hipStream_t st) {
  if (d != 32 * H) return LIME_ERR_UNSUPPORTED;
#define LIME_CS(E, HH) \
  if (ell == E && H == HH) return launch_cs_mfma<E, HH, I8>(cache, qscale, n_items, lp, ids, off, B, total_M, out, bad, st);
  LIME_CS(32, 1) LIME_CS(32, 2) LIME_CS(32, 4) LIME_CS(32, 8)
  LIME_CS(64, 1) LIME_CS(64, 2) LIME_CS(64, 4) LIME_CS(64, 8)
#undef LIME_CS
  return LIME_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------------------
// lime_xor_fwd planning
// ---------------------------------------------------------------------------
struct XorPlan {
  bool mfma = false;       // matrix-core path
  bool resident = false;   // matrix-core, one workgroup per user holding all rows
  int64_t nlr = 0, R = 0;  // link rows, all rows
  int64_t R_pad = 0;       // rows of the QK / packed-V buffers (matrix-core path)
  int S = 1;               // generic path: history splits per user
  int64_t chunk = 1;       // history rows per split
  int64_t G = 0;           // matrix-core path: split slots (an upper bound on the splits)
  size_t o_x = 0, o_qkv = 0, o_v = 0, o_y = 0, o_h = 0, o_part = 0, o_soff = 0, o_suser = 0, total = 0;
  size_t o_ln = 0;         // matrix-core path, d = 256: LayerNorm rows of the next layer [R, d]
  size_t o_lops = 0;       // matrix-core path, d = 256: the link operands of every (user, head)
};

lime_status_t check_sizes(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d, int32_t heads,
                          int32_t d_ff, int64_t total_N, int32_t max_N) {
  if (dtype != LIME_F32 && dtype != LIME_BF16) return fail(LIME_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
  if (B < 1) return fail(LIME_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  if (ell < 1) return fail(LIME_ERR_INVALID_ARG, "ell must be >= 1 (got %d)", ell);
  if (d < 1 || heads < 1) return fail(LIME_ERR_INVALID_ARG, "d and heads must be >= 1");
  if (d % heads != 0) return fail(LIME_ERR_INVALID_ARG, "d (%d) must be a multiple of heads (%d)", d, heads);
  if (d_ff < 1) return fail(LIME_ERR_INVALID_ARG, "d_ff must be >= 1");
  if (total_N < 0 || max_N < 0) return fail(LIME_ERR_INVALID_ARG, "total_N and max_N must be >= 0");
  // (row blocks of 16 are counted in 32 bits on the device)
  if (total_N > (int64_t(1) << 34)) return fail(LIME_ERR_UNSUPPORTED, "total_N above 2^34 rows is unsupported");
  if (ell > 256) return fail(LIME_ERR_UNSUPPORTED, "ell > 256 unsupported (got %d)", ell);
  if (d % 8 != 0 || d > 1024) return fail(LIME_ERR_UNSUPPORTED, "d must be a multiple of 8 and <= 1024 (got %d)", d);
  if (d_ff % 8 != 0 || d_ff > 4096) return fail(LIME_ERR_UNSUPPORTED, "d_ff must be a multiple of 8 and <= 4096 (got %d)", d_ff);
  if (!dh_supported(d / heads)) return fail(LIME_ERR_UNSUPPORTED, "d/heads must be 16, 32, 64 or 128 (got %d)", d / heads);
  return LIME_OK;
}

// shapes served by the matrix-core user-side kernels
bool xor_mfma_ok(lime_dtype_t dtype, int ell, int d, int heads, int d_ff) {
  return dtype == LIME_BF16 && d == 32 * heads && (ell == 32 || ell == 64) &&
         (d == 64 || d == 128 || d == 256) && d_ff == d;
}

// the user-side variant a call runs (LIME-XOR, LIME-MHA, LIME-XOR+Window)
struct VariantArgs {
  bool links_only = false;  // LIME-MHA: history rows are never updated
  int half = 0;             // LIME-XOR+Window: neighbours on each side (0: none)
  // candidate scoring inside the user-resident kernel (score.ids == nullptr:
  // none); *scored is set when the launch took it
  mfma::ScoreArgs score;
  bool* scored = nullptr;
};

// widest window the matrix-core kernels serve for this ell
int mfma_max_half(int ell) { return (mfma::win_nkw(ell) - 32) / 2; }

XorPlan plan_xor(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d, int32_t heads,
                 int32_t d_ff, int64_t total_N, int32_t max_N, bool allow_mfma = true) {
  XorPlan p;
  const size_t es = dtype == LIME_F32 ? 4 : 2;
  p.mfma = allow_mfma && xor_mfma_ok(dtype, ell, d, heads, d_ff);
  if (p.mfma && d <= 128) {
    const int64_t RT = (ell + static_cast<int64_t>(max_N) + 31) / 32 * 32;
    const int64_t per_row = (d + 4) * 4 + (2 * d + 8) * 2 + d * 2 + (d + 8) * 2;
    const int64_t wbytes = d <= 64 ? static_cast<int64_t>(7) * d * (d + 8) * 2 : 0;
    p.resident = RT * per_row + wbytes <= 160 * 1024;
  }
  p.nlr = static_cast<int64_t>(B) * ell;
  p.R = p.nlr + total_N;
  const int dh = d / heads;
  if (p.mfma) {
    // splits of equal row count over all histories (a user's last one
    // shorter): about 2048 (split, head) waves, i.e. one 8-wave workgroup
    // per CU; at least 32 rows each where the history rows' projection is
    // fused into the attention (d <= 128: a split then carries that
    // projection too), 64 otherwise
    int64_t c = (total_N * heads + 2047) / 2048;
    c = (c + 31) / 32 * 32;
    const int64_t cmin = d <= 128 ? 32 : 64;
    p.chunk = c < cmin ? cmin : c;
    // >= sum over users of max(1, ceil((n_b + u0 % 8) / chunk)) (the split
    // grid is anchored at the 8-aligned row below each user's first row)
    p.G = (total_N + 7 * static_cast<int64_t>(B) + p.chunk - 1) / p.chunk + B;
  } else {
    int64_t S = (static_cast<int64_t>(max_N) + 511) / 512;
    if (S < 1) S = 1;
    if (S > 64) S = 64;
    p.S = static_cast<int>(S);
    p.chunk = (static_cast<int64_t>(max_N) + S - 1) / S;
    if (p.chunk < 1) p.chunk = 1;
  }
  size_t off = 0;
  if (p.mfma) {
    p.R_pad = (p.R + 32 + 31) / 32 * 32;
    p.o_x = off;    off = up256(off + static_cast<size_t>(p.R) * d * es);
    p.o_qkv = off;  off = up256(off + static_cast<size_t>(p.R_pad) * 2 * d * es);
    p.o_v = off;    off = up256(off + static_cast<size_t>(p.R_pad) * d * es);
    p.o_y = off;    off = up256(off + static_cast<size_t>(p.R) * d * es);
    p.o_part = off; off = up256(off + static_cast<size_t>(p.G) * heads * ell * mfma::PART_LD * 4);
    p.o_soff = off; off = up256(off + static_cast<size_t>(B + 1) * 4);
    p.o_suser = off; off = up256(off + static_cast<size_t>(p.G) * 4);
    if (d == 256) {
      p.o_ln = off;  off = up256(off + static_cast<size_t>(p.R) * d * es);
      // f16 registers of one wave: 2 (ell / 16) + 2 (ell / 32) of 64 lanes x 16 bytes
      const size_t nreg = static_cast<size_t>(2 * (ell / 16) + 2 * (ell / 32));
      p.o_lops = off; off = up256(off + static_cast<size_t>(B) * heads * nreg * 1024);
    }
  } else {
    p.o_x = off;    off = up256(off + static_cast<size_t>(p.R) * d * es);
    p.o_qkv = off;  off = up256(off + static_cast<size_t>(p.R) * 3 * d * es);
    p.o_y = off;    off = up256(off + static_cast<size_t>(p.R) * d * es);
    p.o_h = off;    off = up256(off + static_cast<size_t>(p.R) * d_ff * es);
    p.o_part = off; off = up256(off + static_cast<size_t>(B) * heads * p.S * ell * (dh + 2) * 4);
  }
  p.total = off;
  return p;
}

int max_dynamic_lds() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 65536;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
    return 65536;
  return v;
}

template <int ELL, int D, int NKW, bool SC = false>
void launch_resident(int B, size_t lds, hipStream_t st, const void* links_ctx, const void* hist,
                     const int64_t* off, int64_t total_N, int RT, int layers, const mfma::LayerSet& ls,
                     float scale, lime_phi_t phi, void* links_pers, void* hist_out, const VariantArgs& va) {
  auto k = mfma::xor_fwd_resident<ELL, D, NKW, SC>;
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               160 * 1024) == hipSuccess;
  (void)attr;
  LIME_LAUNCH(SC ? "xor_fwd_resident_score" : NKW ? "xor_fwd_resident_window" : "xor_fwd_resident", k, dim3(B), dim3(mfma::ResCfg<ELL, D>::NT), lds, st, static_cast<const bf16_t*>(links_ctx),
                     static_cast<const bf16_t*>(hist), off, total_N, RT, layers, ls, scale,
                     static_cast<int>(phi), static_cast<bf16_t*>(links_pers),
                     static_cast<bf16_t*>(hist_out), va.links_only ? 1 : 0, va.half, va.score);
}

// user-resident kernel: one workgroup per user, all layers, when the rows fit
template <int ELL, int D>
bool run_xor_resident(const XorPlan& P, lime_phi_t phi, float scale, int B, int layers,
                      const void* links_ctx, const void* hist, const int64_t* off, int64_t total_N,
                      int32_t max_N, const lime_layer_weights_t* w, void* links_pers, void* hist_out,
                      const VariantArgs& va, hipStream_t st, lime_status_t* status) {
  if constexpr (D > 128) {
    return false;
  } else {
  if (layers > mfma::RES_MAX_LAYERS) return false;
  const int RT = static_cast<int>((ELL + static_cast<int64_t>(max_N) + 31) / 32 * 32);
  const size_t lds = mfma::ResCfg<ELL, D>::lds_bytes(RT);
  static const int limit = max_dynamic_lds();
  if (lds > static_cast<size_t>(limit) || lds > 160 * 1024) return false;
  mfma::LayerSet ls{};
  for (int l = 0; l < layers; ++l) {
    ls.p[l][0] = static_cast<const bf16_t*>(w[l].w_qkv);
    ls.p[l][1] = static_cast<const bf16_t*>(w[l].w_o);
    ls.p[l][2] = static_cast<const bf16_t*>(w[l].w_gate);
    ls.p[l][3] = static_cast<const bf16_t*>(w[l].w_up);
    ls.p[l][4] = static_cast<const bf16_t*>(w[l].w_down);
  }
  const bool score = va.score.ids != nullptr && va.half == 0 && !va.links_only;
  if (va.half > 0)
    launch_resident<ELL, D, mfma::win_nkw(ELL)>(B, lds, st, links_ctx, hist, off, total_N, RT, layers, ls, scale,
                                                 phi, links_pers, hist_out, va);
  else if (score)
    launch_resident<ELL, D, 0, true>(B, lds, st, links_ctx, hist, off, total_N, RT, layers, ls, scale, phi,
                                     links_pers, hist_out, va);
  else
    launch_resident<ELL, D, 0>(B, lds, st, links_ctx, hist, off, total_N, RT, layers, ls, scale, phi,
                               links_pers, hist_out, va);
  hipError_t e = hipGetLastError();
  *status = (e == hipSuccess) ? ok() : fail(LIME_ERR_HIP, "user-resident xor: %s", hipGetErrorString(e));
  if (va.scored != nullptr && score) *va.scored = true;
  (void)P;
  return true;
  }
}

// matrix-core user side: per layer QKV projection, XOR attention, split
// combine, fused post-attention block
template <int ELL, int D>
lime_status_t run_xor_mfma(const XorPlan& P, lime_phi_t phi, float scale, int B, int layers,
                           const void* links_ctx, const void* hist, const int64_t* off,
                           int64_t total_N, int32_t max_N, const lime_layer_weights_t* w,
                           void* links_pers, void* hist_out, const VariantArgs& va, char* ws,
                           hipStream_t st) {
  if (P.resident) {
    lime_status_t status = LIME_OK;
    if (run_xor_resident<ELL, D>(P, phi, scale, B, layers, links_ctx, hist, off, total_N, max_N, w,
                                 links_pers, hist_out, va, st, &status))
      return status;
  }
  constexpr int H = D / 32;
  constexpr int RPW = D >= 256 ? 16 : 32;
  bf16_t* X = reinterpret_cast<bf16_t*>(ws + P.o_x);
  bf16_t* QK = reinterpret_cast<bf16_t*>(ws + P.o_qkv);
  bf16_t* Vp = reinterpret_cast<bf16_t*>(ws + P.o_v);
  bf16_t* Y = reinterpret_cast<bf16_t*>(ws + P.o_y);
  float* part = reinterpret_cast<float*>(ws + P.o_part);
  int32_t* soff = reinterpret_cast<int32_t*>(ws + P.o_soff);
  int32_t* suser = reinterpret_cast<int32_t*>(ws + P.o_suser);
  const int64_t nlr = P.nlr, R = P.R;
  const Rows Xws{X, X + nlr * D, nlr, D};
  // d = 256 without the window: the projection runs inside the attention,
  // from the LayerNorm rows the previous post block stored (the first layer
  // normalises the input rows itself).  LIME-MHA runs every layer in the
  // links-only form of the last LIME-XOR layer; its history rows, never
  // updated, keep the first layer's LayerNorm rows.
  const bool fused_h = D == 256 && va.half == 0;
  bf16_t* LNr = fused_h ? reinterpret_cast<bf16_t*>(ws + P.o_ln) : nullptr;
  const Rows LNrows{LNr, LNr + nlr * D, nlr, D};
  void* lops = fused_h ? ws + P.o_lops : nullptr;
  // the splits of every layer's attention
  LIME_LAUNCH("split_plan", mfma::split_plan, dim3(1), dim3(mfma::SPLIT_PLAN_NT), 0, st, off, B, total_N, P.chunk,
                     soff, suser, static_cast<int>(P.G));
  LIME_CHECK_LAUNCH("split plan");
  // Q|K and Y are head-planar in the workspace (see the kernels' Lay)
  // the projections store Q times the logit scale in log2 units; the
  // attention kernels then work with base-2 exponentials
  const float qs = scale * mfma::LOG2E;
  for (int l = 0; l < layers; ++l) {
    const bool last = (l == layers - 1);
    const bool full = !va.links_only && (!last || hist_out != nullptr);
    const int64_t rows_post = full ? R : nlr;
    // LIME-MHA never updates history rows: every layer reads the input E
    const Rows Xin = (l == 0) ? Rows{const_cast<void*>(links_ctx), const_cast<void*>(hist), nlr, D}
                     : va.links_only ? Rows{X, const_cast<void*>(hist), nlr, D} : Xws;
    const Rows Xout = last ? Rows{links_pers, hist_out, nlr, D} : Xws;
    // history rows need Q only for their own attention (the E-branch); the
    // links always need it
    const int64_t q_rows = full ? P.R_pad : nlr;
    // d <= 128 without the window: the projection runs inside the attention
    // kernel
    const bool fused = (D <= 128 && !(va.half > 0 && full)) || fused_h;
    if (!fused) {
      if constexpr (D <= 128) {
        // weights staged in LDS, persistent workgroups (one per CU)
        auto k = mfma::qkv_proj_lds<D>;
        constexpr size_t lds = mfma::QkvLds<D>::lds_bytes;
        static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     static_cast<int>(lds)) == hipSuccess;
        (void)attr;
        static const int per_cu = blocks_per_cu_lds(k, 64 * mfma::QkvLds<D>::NW, lds);
        const int64_t nproj = P.R_pad;
        const int64_t nblk = nproj / 32;
        int64_t grid = static_cast<int64_t>(cu_count()) * per_cu;
        const int64_t need = (nblk + mfma::QkvLds<D>::NW - 1) / mfma::QkvLds<D>::NW;
        if (grid > need) grid = need;
        LIME_LAUNCH("qkv_proj_lds", k, dim3(static_cast<unsigned>(grid)), dim3(64 * mfma::QkvLds<D>::NW), lds, st, Xin, R,
                           P.R_pad, nproj, static_cast<const bf16_t*>(w[l].w_qkv), QK, Vp, qs, q_rows);
      } else {
        // weights streamed through LDS, persistent workgroups
        auto k = mfma::qkv_proj_stream<D>;
        constexpr size_t lds = mfma::StreamCfg<D>::lds_bytes;
        static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     static_cast<int>(lds)) == hipSuccess;
        (void)attr;
        static const int per_cu = blocks_per_cu_lds(k, mfma::StreamCfg<D>::NT, lds);
        const int64_t ntiles = (P.R_pad + mfma::StreamCfg<D>::TILE - 1) / mfma::StreamCfg<D>::TILE;
        int64_t grid = static_cast<int64_t>(cu_count()) * per_cu;
        if (grid > ntiles) grid = ntiles;
        LIME_LAUNCH("qkv_proj_stream", k, dim3(static_cast<unsigned>(grid)), dim3(mfma::StreamCfg<D>::NT), lds, st, Xin, R,
                           P.R_pad, static_cast<const bf16_t*>(w[l].w_qkv), QK, Vp, qs, q_rows);
      }
      LIME_CHECK_LAUNCH("qkv projection (mfma)");
    }
    {
      // one workgroup per (split slot, head group); slots past the last
      // split return at once
      const dim3 grid(static_cast<unsigned>(P.G));
      // the windowed form runs at most 4 heads per workgroup (registers)
      constexpr int HBW = H > 4 ? 4 : H;
      const dim3 grid_w(static_cast<unsigned>(P.G * (H / HBW)));
      if (fused_h) {
        if constexpr (D == 256) {
          using FC = mfma::FusedHCfg<ELL>;
          // (the same signature for both forms: each sets its own LDS limit)
          auto kf = mfma::xor_attn_h<ELL, false, true>;
          auto kl = mfma::xor_attn_h<ELL, false, false>;
          auto pf = mfma::link_qkv_h<ELL, true>;
          auto pl = mfma::link_qkv_h<ELL, false>;
          static const bool attr_f = hipFuncSetAttribute(reinterpret_cast<const void*>(kf),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         static_cast<int>(FC::lds_bytes)) == hipSuccess;
          static const bool attr_l = hipFuncSetAttribute(reinterpret_cast<const void*>(kl),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         static_cast<int>(FC::lds_bytes)) == hipSuccess;
          (void)attr_f;
          (void)attr_l;
          if (l == 0) {
            // the first layer's LayerNorm rows
            LIME_LAUNCH("ln_rows", mfma::ln_rows_kernel<D>, dim3(static_cast<unsigned>(cu_count() * 8)), dim3(256), 0,
                        st, Xin, R, LNr);
            LIME_CHECK_LAUNCH("layer-0 LayerNorm rows");
          }
          // the link operands once per (user, head), then the attention
          const int64_t pgrid = full ? mfma::LinkQkvCfg<ELL, true>::grid(B) : mfma::LinkQkvCfg<ELL, false>::grid(B);
          LIME_LAUNCH("link_qkv_h", full ? pf : pl, dim3(static_cast<unsigned>(pgrid)), dim3(64), 0, st, LNrows,
                      static_cast<const bf16_t*>(w[l].w_qkv), lops, qs);
          LIME_CHECK_LAUNCH("link operands (d = 256)");
          LIME_LAUNCH("xor_attn_h", full ? kf : kl, dim3(static_cast<unsigned>(FC::grid(P.G))), dim3(64 * FC::NW),
                      FC::lds_bytes, st, LNrows, static_cast<const bf16_t*>(w[l].w_qkv), lops, Y, part, off, soff,
                      suser, B, static_cast<int>(P.G), P.chunk, total_N, static_cast<int>(phi));
        }
      } else if (fused) {
        if constexpr (D <= 128) {
          using FC = mfma::FusedCfg<ELL, H>;
          auto k = mfma::xor_attn_qkv<ELL, H>;
          static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(FC::lds_bytes)) == hipSuccess;
          (void)attr;
          const dim3 grid_f(static_cast<unsigned>((P.G + FC::SPW - 1) / FC::SPW));
          LIME_LAUNCH("xor_attn_qkv", k, grid_f, dim3(64 * FC::NW), FC::lds_bytes, st, Xin,
                             static_cast<const bf16_t*>(w[l].w_qkv), Y, part, off, soff, suser, B,
                             static_cast<int>(P.G), P.chunk, total_N, static_cast<int>(phi), full ? 1 : 0, qs);
        }
      } else if (va.half > 0 && full)
        LIME_LAUNCH("xor_attn_window", (mfma::xor_attn<ELL, H, mfma::win_nkw(ELL), HBW>), grid_w, dim3(64 * HBW), 0, st, QK,
                           Vp, Y, part, off, soff, suser, B, P.chunk, total_N, static_cast<int>(phi), 1, va.half,
                           P.R_pad);
      else
        LIME_LAUNCH("xor_attn", (mfma::xor_attn<ELL, H>), grid, dim3(64 * H), 0, st, QK, Vp, Y, part, off, soff, suser,
                           B, P.chunk, total_N, static_cast<int>(phi), full ? 1 : 0, 0, P.R_pad);
    }
    LIME_CHECK_LAUNCH("xor attention (mfma)");
    {
      const int64_t n = static_cast<int64_t>(B) * H * ELL * 4 * mfma::CSG;
      LIME_LAUNCH("xor_combine", (mfma::xor_combine<ELL>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                         part, soff, Y, B, H, R * 32);
      LIME_CHECK_LAUNCH("xor combine");
    }
    const int64_t pw = (rows_post + RPW - 1) / RPW;
    if constexpr (D <= 128) {
      auto k = mfma::post_block_lds<D, D, RPW>;
      constexpr size_t lds = mfma::PostLds<D, D>::lds_bytes;
      static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   static_cast<int>(lds)) == hipSuccess;
      (void)attr;
      static const int per_cu = blocks_per_cu_lds(k, 64 * mfma::PostLds<D, D>::NW, lds);
      int64_t grid = static_cast<int64_t>(cu_count()) * per_cu;
      const int64_t need = (pw + mfma::PostLds<D, D>::NW - 1) / mfma::PostLds<D, D>::NW;
      if (grid > need) grid = need;
      LIME_LAUNCH("post_block_lds", k, dim3(static_cast<unsigned>(grid)), dim3(64 * mfma::PostLds<D, D>::NW), lds, st, Y, R,
                         Xin, Xout, rows_post, static_cast<const bf16_t*>(w[l].w_o),
                         static_cast<const bf16_t*>(w[l].w_gate), static_cast<const bf16_t*>(w[l].w_up),
                         static_cast<const bf16_t*>(w[l].w_down));
    } else {
      (void)pw;
      auto k = mfma::post_block_stream<D>;
      using PC = mfma::PostStreamCfg<D>;
      constexpr size_t lds = PC::lds_bytes;
      static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   static_cast<int>(lds)) == hipSuccess;
      (void)attr;
      static const int per_cu = blocks_per_cu_lds(k, PC::NT, lds);
      // every workgroup gets at least one 16-row block
      const int64_t nblk = (rows_post + 15) / 16;
      int64_t grid = static_cast<int64_t>(cu_count()) * per_cu;
      if (grid > nblk) grid = nblk;
      // the next layer's LayerNorm rows for the fused attention
      const Rows Hout = (fused_h && !last) ? LNrows : Rows{nullptr, nullptr, 0, 0};
      LIME_LAUNCH("post_block_stream", k, dim3(static_cast<unsigned>(grid)), dim3(PC::NT), lds, st, static_cast<const bf16_t*>(Y), R, Xin,
                         Xout, rows_post, static_cast<const bf16_t*>(w[l].w_o),
                         static_cast<const bf16_t*>(w[l].w_gate), static_cast<const bf16_t*>(w[l].w_up),
                         static_cast<const bf16_t*>(w[l].w_down), Hout);
    }
    LIME_CHECK_LAUNCH("post-attention block (mfma)");
  }
  return ok();
}

lime_status_t dispatch_xor_mfma(const XorPlan& P, lime_phi_t phi, float scale, int B, int ell, int d,
                                int layers, const void* links_ctx, const void* hist,
                                const int64_t* off, int64_t total_N, int32_t max_N,
                                const lime_layer_weights_t* w,
                                void* links_pers, void* hist_out, const VariantArgs& va, char* ws,
                                hipStream_t st) {
#define LIME_XM(E, DD) \
  if (ell == E && d == DD) return run_xor_mfma<E, DD>(P, phi, scale, B, layers, links_ctx, hist, off, total_N, max_N, w, links_pers, hist_out, va, ws, st);
  LIME_XM(32, 64) LIME_XM(32, 128) LIME_XM(32, 256)
  LIME_XM(64, 64) LIME_XM(64, 128) LIME_XM(64, 256)
#undef LIME_XM
  return fail(LIME_ERR_UNSUPPORTED, "no matrix-core user-side kernel for ell=%d d=%d", ell, d);
}

template <typename T, int DH>
lime_status_t run_xor_generic(const XorPlan& P, lime_phi_t phi, float scale, int B, int ell,
                              int d, int H, int layers, int d_ff, const void* links_ctx,
                              const void* hist, const int64_t* off, int64_t total_N,
                              const lime_layer_weights_t* w, void* links_pers, void* hist_out,
                              const VariantArgs& va, char* ws, hipStream_t st) {
  using namespace gen;
  T* X = reinterpret_cast<T*>(ws + P.o_x);
  T* QKV = reinterpret_cast<T*>(ws + P.o_qkv);
  T* Y = reinterpret_cast<T*>(ws + P.o_y);
  T* Hm = reinterpret_cast<T*>(ws + P.o_h);
  float* part = reinterpret_cast<float*>(ws + P.o_part);
  const int64_t nlr = P.nlr, R = P.R;
  const Rows Xws{X, X + nlr * d, nlr, d};
  const Rows QKVr{QKV, QKV + nlr * 3 * d, nlr, 3 * static_cast<int64_t>(d)};
  const Rows Yr{Y, Y + nlr * d, nlr, d};
  const Rows Hr{Hm, Hm + nlr * d_ff, nlr, d_ff};
  const Rows none{nullptr, nullptr, 0, 0};
  const dim3 blk(256);
  auto gx = [](int64_t rows) { return static_cast<unsigned>((rows + GB_M - 1) / GB_M); };
  auto gy = [](int cols) { return static_cast<unsigned>((cols + GB_N - 1) / GB_N); };

  for (int l = 0; l < layers; ++l) {
    const bool last = (l == layers - 1);
    const bool full = !va.links_only && (!last || hist_out != nullptr);
    const int64_t rows_post = full ? R : nlr;
    const Rows Xin = (l == 0) ? Rows{const_cast<void*>(links_ctx), const_cast<void*>(hist), nlr, d}
                     : va.links_only ? Rows{X, const_cast<void*>(hist), nlr, d} : Xws;
    const Rows Xfinal = last ? Rows{links_pers, hist_out, nlr, d} : Xws;
    const T* Wqkv = static_cast<const T*>(w[l].w_qkv);

    LIME_LAUNCH("gen::qkv_proj", (gemm_rows<T, true, EPI_STORE>), dim3(gx(R), gy(3 * d)), blk, 0, st, Xin,
                       int64_t(0), R, d, Wqkv, nullptr, 3 * d, none, QKVr);
    LIME_CHECK_LAUNCH("qkv projection");
    LIME_LAUNCH("gen::xor_attn", (xor_attn<T, DH>), dim3(B, H, P.S), blk, 0, st, QKV, Y, part, off, B, ell,
                       d, H, P.S, P.chunk, total_N, scale, static_cast<int>(phi), full ? 1 : 0, va.half);
    LIME_CHECK_LAUNCH("xor attention");
    {
      const int64_t n = static_cast<int64_t>(B) * H * ell * DH;
      LIME_LAUNCH("gen::xor_combine", (xor_combine<T, DH>), dim3(static_cast<unsigned>((n + 255) / 256)), blk, 0,
                         st, part, Y, B, ell, d, H, P.S, static_cast<int64_t>(d), static_cast<int64_t>(DH));
      LIME_CHECK_LAUNCH("xor combine");
    }
    LIME_LAUNCH("gen::out_proj", (gemm_rows<T, false, EPI_RESID>), dim3(gx(rows_post), gy(d)), blk, 0, st,
                       Yr, int64_t(0), rows_post, d, static_cast<const T*>(w[l].w_o), nullptr, d,
                       Xin, Xws);
    LIME_CHECK_LAUNCH("output projection");
    LIME_LAUNCH("gen::mlp_up", (gemm_rows<T, true, EPI_SWIGLU>), dim3(gx(rows_post), gy(d_ff)), blk, 0,
                       st, Xws, int64_t(0), rows_post, d, static_cast<const T*>(w[l].w_gate),
                       static_cast<const T*>(w[l].w_up), d_ff, none, Hr);
    LIME_CHECK_LAUNCH("gated mlp up");
    LIME_LAUNCH("gen::mlp_down", (gemm_rows<T, false, EPI_RESID>), dim3(gx(rows_post), gy(d)), blk, 0, st,
                       Hr, int64_t(0), rows_post, d_ff, static_cast<const T*>(w[l].w_down),
                       nullptr, d, Xws, Xfinal);
    LIME_CHECK_LAUNCH("gated mlp down");
  }
  return ok();
}

template <typename T>
lime_status_t dispatch_xor_generic(int dh, const XorPlan& P, lime_phi_t phi, float scale, int B,
                                   int ell, int d, int H, int layers, int d_ff,
                                   const void* links_ctx, const void* hist, const int64_t* off,
                                   int64_t total_N, const lime_layer_weights_t* w,
                                   void* links_pers, void* hist_out, const VariantArgs& va, char* ws,
                                   hipStream_t st) {
  switch (dh) {
    case 16: return run_xor_generic<T, 16>(P, phi, scale, B, ell, d, H, layers, d_ff, links_ctx, hist, off, total_N, w, links_pers, hist_out, va, ws, st);
    case 32: return run_xor_generic<T, 32>(P, phi, scale, B, ell, d, H, layers, d_ff, links_ctx, hist, off, total_N, w, links_pers, hist_out, va, ws, st);
    case 64: return run_xor_generic<T, 64>(P, phi, scale, B, ell, d, H, layers, d_ff, links_ctx, hist, off, total_N, w, links_pers, hist_out, va, ws, st);
    case 128: return run_xor_generic<T, 128>(P, phi, scale, B, ell, d, H, layers, d_ff, links_ctx, hist, off, total_N, w, links_pers, hist_out, va, ws, st);
  }
  return fail(LIME_ERR_UNSUPPORTED, "d_h %d", dh);
}

// The workspace of lime_xor_fwd_noalloc: a fixed device array, one copy per
// GPU, held until the process ends.  Host code must never pass `scratch`
// itself to a kernel or a runtime call (in host code the name is a host-side
// stand-in, not a device address): its address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[LIME_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address, looked up on its first use
lime_status_t scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LIME_ERR_HIP, "noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(LIME_ERR_UNSUPPORTED, "noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(LIME_ERR_HIP, "noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LIME_OK;
}

}  // namespace

extern "C" {

const char* lime_status_string(lime_status_t s) {
  switch (s) {
    case LIME_OK: return "LIME_OK";
    case LIME_ERR_INVALID_ARG: return "LIME_ERR_INVALID_ARG";
    case LIME_ERR_UNSUPPORTED: return "LIME_ERR_UNSUPPORTED";
    case LIME_ERR_WORKSPACE: return "LIME_ERR_WORKSPACE";
    case LIME_ERR_HIP: return "LIME_ERR_HIP";
  }
  return "LIME_ERR_UNKNOWN";
}

const char* lime_last_error(void) { return g_err.c_str(); }

lime_status_t lime_trace_begin(int32_t capacity) {
  if (capacity < 1) return fail(LIME_ERR_INVALID_ARG, "trace capacity must be >= 1 (got %d)", capacity);
  std::lock_guard<std::mutex> lk(g_trace.m);
  if (g_trace.on.load(std::memory_order_relaxed)) return fail(LIME_ERR_INVALID_ARG, "a trace is already open");
  std::vector<hipEvent_t> ev(2 * static_cast<size_t>(capacity), nullptr);
  for (size_t i = 0; i < ev.size(); ++i) {
    if (hipEventCreate(&ev[i]) != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return fail(LIME_ERR_HIP, "trace: hipEventCreate failed");
    }
  }
  g_trace.ev.swap(ev);
  g_trace.name.assign(static_cast<size_t>(capacity), nullptr);
  g_trace.n = 0;
  g_trace.dropped = 0;
  g_trace.on.store(true, std::memory_order_release);
  return ok();
}

int32_t lime_trace_end(const char** names, float* ms, int32_t cap, int32_t* dropped) {
  std::lock_guard<std::mutex> lk(g_trace.m);
  if (!g_trace.on.load(std::memory_order_relaxed)) {
    fail(LIME_ERR_INVALID_ARG, "no trace is open");
    return -1;
  }
  g_trace.on.store(false, std::memory_order_release);
  int32_t n = g_trace.n;
  bool waited = true;
  for (int32_t i = 0; i < n; ++i) {
    float t = 0.f;
    if (hipEventSynchronize(g_trace.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]) != hipSuccess)
      waited = false;
    if (i < cap) {
      if (names) names[i] = g_trace.name[i];
      if (ms) ms[i] = t;
    }
  }
  if (dropped) *dropped = g_trace.dropped;
  for (hipEvent_t e : g_trace.ev) (void)hipEventDestroy(e);
  g_trace.ev.clear();
  g_trace.name.clear();
  g_trace.n = 0;
  if (!waited) {
    fail(LIME_ERR_HIP, "trace: waiting for a traced launch failed");
    return -1;
  }
  ok();
  return n;
}

size_t lime_xor_fwd_workspace_size(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                                   int32_t heads, int32_t d_ff, int64_t total_N, int32_t max_N) {
  if (check_sizes(dtype, B, ell, d, heads, d_ff, total_N, max_N) != LIME_OK) return 0;
  // the matrix-core layout, or the generic one a variant may fall back to
  const size_t a = plan_xor(dtype, B, ell, d, heads, d_ff, total_N, max_N, true).total;
  const size_t b = plan_xor(dtype, B, ell, d, heads, d_ff, total_N, max_N, false).total;
  return a > b ? a : b;
}

int32_t lime_xor_fwd_plan(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d, int32_t heads,
                          int32_t layers, int32_t d_ff, int64_t total_N, int32_t max_N,
                          int32_t with_hist, char* buf, size_t buf_len) {
  if (check_sizes(dtype, B, ell, d, heads, d_ff, total_N, max_N) != LIME_OK || layers < 1) return 0;
  const XorPlan P = plan_xor(dtype, B, ell, d, heads, d_ff, total_N, max_N);
  const bool resident = P.mfma && P.resident && d <= 128 && layers <= mfma::RES_MAX_LAYERS;
  int32_t launches;
  char line[512];
  if (resident) {
    launches = 1;
    snprintf(line, sizeof(line), "user-resident: 1 launch for %d layers, one workgroup per user", layers);
  } else if (P.mfma && d <= 128) {
    launches = 3 * layers + 1;
    snprintf(line, sizeof(line),
             "streaming matrix-core: a split plan, then 3 launches per layer (qkv + xor_attn fused, "
             "combine, post); splits of %lld history rows, at most %lld splits",
             static_cast<long long>(P.chunk), static_cast<long long>(P.G));
  } else if (P.mfma) {
    launches = 4 * layers + 2;
    snprintf(line, sizeof(line),
             "streaming matrix-core: a split plan and the first layer's LayerNorm rows, then 4 launches per "
             "layer (link_qkv_h: the link rows' Q, K, V once per user and head; xor_attn_h: the attention with the "
             "history rows' projection fused in, from LayerNorm rows the post block stores; combine; post); "
             "splits of %lld history rows, at most %lld splits",
             static_cast<long long>(P.chunk), static_cast<long long>(P.G));
  } else {
    launches = 6 * layers;
    snprintf(line, sizeof(line),
             "generic: 6 launches per layer, %d splits per user of %lld rows", P.S,
             static_cast<long long>(P.chunk));
  }
  (void)with_hist;
  if (buf && buf_len > 0) snprintf(buf, buf_len, "%s", line);
  return launches;
}

lime_status_t lime_xor_fwd(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                           int32_t ell, int32_t d, int32_t heads, int32_t layers, int32_t d_ff,
                           const void* links_ctx, const void* hist, const int64_t* hist_offsets,
                           int64_t total_N, int32_t max_N, const lime_layer_weights_t* w,
                           void* links_pers, void* hist_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return lime_xor_fwd_variant(LIME_VARIANT_XOR, 0, dtype, phi, scale, B, ell, d, heads, layers, d_ff,
                              links_ctx, hist, hist_offsets, total_N, max_N, w, links_pers, hist_out,
                              workspace, workspace_bytes, stream);
}

// score != nullptr: also score the candidates inside the user-resident
// kernel when that path runs (*scored tells whether it did)
static lime_status_t xor_fwd_impl(lime_variant_t variant, int32_t window, lime_dtype_t dtype,
                                  lime_phi_t phi, float scale, int32_t B, int32_t ell, int32_t d,
                                  int32_t heads, int32_t layers, int32_t d_ff,
                                  const void* links_ctx, const void* hist,
                                  const int64_t* hist_offsets, int64_t total_N, int32_t max_N,
                                  const lime_layer_weights_t* w, void* links_pers,
                                  void* hist_out, void* workspace, size_t workspace_bytes,
                                  void* stream, const mfma::ScoreArgs* score, bool* scored) {
  lime_status_t st = check_sizes(dtype, B, ell, d, heads, d_ff, total_N, max_N);
  if (st != LIME_OK) return st;
  VariantArgs va;
  if (score != nullptr) {
    va.score = *score;
    va.scored = scored;
  }
  switch (variant) {
    case LIME_VARIANT_XOR:
      if (window != 0) return fail(LIME_ERR_INVALID_ARG, "window must be 0 for LIME_VARIANT_XOR");
      break;
    case LIME_VARIANT_MHA:
      if (window != 0) return fail(LIME_ERR_INVALID_ARG, "window must be 0 for LIME_VARIANT_MHA");
      if (hist_out) return fail(LIME_ERR_INVALID_ARG, "LIME_VARIANT_MHA does not update history rows: hist_out must be NULL");
      va.links_only = true;
      break;
    case LIME_VARIANT_XOR_WINDOW:
      if (window < 1 || window > 4096)
        return fail(LIME_ERR_INVALID_ARG, "window must be in [1, 4096] for LIME_VARIANT_XOR_WINDOW (got %d)", window);
      va.half = window;
      break;
    default:
      return fail(LIME_ERR_INVALID_ARG, "bad variant %d", (int)variant);
  }
  if (phi != LIME_PHI_SOFTMAX && phi != LIME_PHI_SILU_MEAN) return fail(LIME_ERR_INVALID_ARG, "bad phi %d", (int)phi);
  if (!std::isfinite(scale)) return fail(LIME_ERR_INVALID_ARG, "scale must be finite");
  if (layers < 1) return fail(LIME_ERR_INVALID_ARG, "layers must be >= 1 (got %d)", layers);
  if (!links_ctx || !hist_offsets || !w || !links_pers) return fail(LIME_ERR_INVALID_ARG, "null pointer argument");
  if (total_N > 0 && !hist) return fail(LIME_ERR_INVALID_ARG, "hist is null but total_N > 0");
  if (!aligned16(links_ctx) || !aligned16(hist) || !aligned16(hist_offsets) ||
      !aligned16(links_pers) || !aligned16(hist_out))
    return fail(LIME_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  for (int l = 0; l < layers; ++l) {
    const lime_layer_weights_t& lw = w[l];
    if (!lw.w_qkv || !lw.w_o || !lw.w_gate || !lw.w_up || !lw.w_down)
      return fail(LIME_ERR_INVALID_ARG, "null weight pointer in layer %d", l);
    if (!aligned16(lw.w_qkv) || !aligned16(lw.w_o) || !aligned16(lw.w_gate) ||
        !aligned16(lw.w_up) || !aligned16(lw.w_down))
      return fail(LIME_ERR_INVALID_ARG, "weights of layer %d not 16-byte aligned", l);
  }
  // windows wider than the matrix-core kernels serve run on the generic ones
  const bool allow_mfma = va.half <= mfma_max_half(ell);
  const XorPlan P = plan_xor(dtype, B, ell, d, heads, d_ff, total_N, max_N, allow_mfma);
  if (!workspace) return fail(LIME_ERR_WORKSPACE, "workspace is null");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LIME_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < P.total)
    return fail(LIME_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, P.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int dh = d / heads;
  if (P.mfma)
    return dispatch_xor_mfma(P, phi, scale, B, ell, d, layers, links_ctx, hist, hist_offsets, total_N,
                             max_N, w, links_pers, hist_out, va, ws, s);
  if (dtype == LIME_F32)
    return dispatch_xor_generic<float>(dh, P, phi, scale, B, ell, d, heads, layers, d_ff, links_ctx,
                                       hist, hist_offsets, total_N, w, links_pers, hist_out, va, ws, s);
  return dispatch_xor_generic<bf16_t>(dh, P, phi, scale, B, ell, d, heads, layers, d_ff, links_ctx,
                                      hist, hist_offsets, total_N, w, links_pers, hist_out, va, ws, s);
}

lime_status_t lime_xor_fwd_variant(lime_variant_t variant, int32_t window, lime_dtype_t dtype,
                                   lime_phi_t phi, float scale, int32_t B, int32_t ell, int32_t d,
                                   int32_t heads, int32_t layers, int32_t d_ff,
                                   const void* links_ctx, const void* hist,
                                   const int64_t* hist_offsets, int64_t total_N, int32_t max_N,
                                   const lime_layer_weights_t* w, void* links_pers,
                                   void* hist_out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return xor_fwd_impl(variant, window, dtype, phi, scale, B, ell, d, heads, layers, d_ff, links_ctx, hist,
                      hist_offsets, total_N, max_N, w, links_pers, hist_out, workspace, workspace_bytes, stream,
                      nullptr, nullptr);
}

lime_status_t lime_xor_fwd_noalloc(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                                   int32_t ell, int32_t d, int32_t heads, int32_t layers, int32_t d_ff,
                                   const void* links_ctx, const void* hist, const int64_t* hist_offsets,
                                   int64_t total_N, int32_t max_N, const lime_layer_weights_t* w,
                                   void* links_pers, void* hist_out, void* stream) {
  lime_status_t st = check_sizes(dtype, B, ell, d, heads, d_ff, total_N, max_N);
  if (st != LIME_OK) return st;
  // the size check comes before the device lookup, so an oversized call
  // touches no GPU state
  const size_t need = lime_xor_fwd_workspace_size(dtype, B, ell, d, heads, d_ff, total_N, max_N);
  if (need > LIME_NOALLOC_SCRATCH_BYTES)
    return fail(LIME_ERR_WORKSPACE, "noalloc: the call needs %zu bytes of workspace, more than the %llu of the "
                "library's scratch array", need, static_cast<unsigned long long>(LIME_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != LIME_OK) return st;
  return xor_fwd_impl(LIME_VARIANT_XOR, 0, dtype, phi, scale, B, ell, d, heads, layers, d_ff, links_ctx, hist,
                      hist_offsets, total_N, max_N, w, links_pers, hist_out, ws, LIME_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr, nullptr);
}

static lime_status_t qk_cache_impl(bool i8, lime_dtype_t dtype, lime_phi_t phi, float scale,
                                   int64_t n_items, int32_t d, int32_t heads, int32_t ell,
                                   const void* items, const void* link_keys, void* cache,
                                   float* qscale, void* stream) {
  if (dtype != LIME_F32 && dtype != LIME_BF16) return fail(LIME_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
  if (phi != LIME_PHI_SOFTMAX && phi != LIME_PHI_SILU_MEAN) return fail(LIME_ERR_INVALID_ARG, "bad phi %d", (int)phi);
  if (!std::isfinite(scale)) return fail(LIME_ERR_INVALID_ARG, "scale must be finite");
  if (n_items < 0 || d < 1 || heads < 1 || ell < 1) return fail(LIME_ERR_INVALID_ARG, "sizes must be positive");
  if (ell > 256) return fail(LIME_ERR_UNSUPPORTED, "ell > 256 unsupported (got %d)", ell);
  if (d % 8 != 0 || d > 1024) return fail(LIME_ERR_UNSUPPORTED, "d must be a multiple of 8 and <= 1024 (got %d)", d);
  if (heads > 65535) return fail(LIME_ERR_UNSUPPORTED, "too many heads");
  if (!link_keys) return fail(LIME_ERR_INVALID_ARG, "link_keys is null");
  if (n_items > 0 && (!items || !cache)) return fail(LIME_ERR_INVALID_ARG, "null pointer argument");
  if (i8 && n_items > 0 && !qscale) return fail(LIME_ERR_INVALID_ARG, "qscale is null");
  if (!aligned16(items) || !aligned16(link_keys) || !aligned16(cache))
    return fail(LIME_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (i8 && (reinterpret_cast<uintptr_t>(qscale) & 3u) != 0)
    return fail(LIME_ERR_INVALID_ARG, "qscale must be 4-byte aligned");
  if (n_items == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LIME_BF16) {
    const lime_status_t r = i8 ? try_qk_mfma<true>(ell, d, heads, items, link_keys, cache, qscale, n_items, scale,
                                                   static_cast<int>(phi), s)
                               : try_qk_mfma<false>(ell, d, heads, items, link_keys, cache, qscale, n_items, scale,
                                                    static_cast<int>(phi), s);
    if (r != LIME_ERR_UNSUPPORTED) return r;
  }
  const dim3 grid(static_cast<unsigned>((n_items + 63) / 64), heads);
  const size_t lds = 64 * static_cast<size_t>(ell) * 4;
#define LIME_QKG(T, I) \
  LIME_LAUNCH("gen::qk_cache", (gen::qk_cache<T, I>), grid, dim3(64), lds, s, static_cast<const T*>(items), \
                     static_cast<const T*>(link_keys), cache, qscale, n_items, d, heads, ell, scale, \
                     static_cast<int>(phi))
  if (dtype == LIME_F32) {
    if (i8) LIME_QKG(float, true); else LIME_QKG(float, false);
  } else {
    if (i8) LIME_QKG(bf16_t, true); else LIME_QKG(bf16_t, false);
  }
#undef LIME_QKG
  LIME_CHECK_LAUNCH("qk cache build");
  return ok();
}

static lime_status_t check_score(bool i8, lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                                 int32_t heads, const void* cache, const float* qscale, int64_t n_items,
                                 const void* links_pers, const int64_t* cand_ids,
                                 const int64_t* cand_offsets, int64_t total_M, void* out,
                                 int32_t* bad_id_count) {
  if (dtype != LIME_F32 && dtype != LIME_BF16) return fail(LIME_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
  if (B < 1 || ell < 1 || d < 1 || heads < 1 || n_items < 0 || total_M < 0)
    return fail(LIME_ERR_INVALID_ARG, "sizes must be positive");
  if (d % heads != 0) return fail(LIME_ERR_INVALID_ARG, "d (%d) must be a multiple of heads (%d)", d, heads);
  if (ell > 256) return fail(LIME_ERR_UNSUPPORTED, "ell > 256 unsupported (got %d)", ell);
  if (!dh_supported(d / heads)) return fail(LIME_ERR_UNSUPPORTED, "d/heads must be 16, 32, 64 or 128 (got %d)", d / heads);
  if (!links_pers || !cand_offsets) return fail(LIME_ERR_INVALID_ARG, "null pointer argument");
  if (total_M > 0 && (!cand_ids || !out)) return fail(LIME_ERR_INVALID_ARG, "null pointer argument");
  if (n_items > 0 && !cache) return fail(LIME_ERR_INVALID_ARG, "cache is null");
  if (i8 && n_items > 0 && !qscale) return fail(LIME_ERR_INVALID_ARG, "qscale is null");
  if (!aligned16(cache) || !aligned16(links_pers) || !aligned16(cand_ids) ||
      !aligned16(cand_offsets) || !aligned16(out))
    return fail(LIME_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(bad_id_count) & 3u) != 0 || (reinterpret_cast<uintptr_t>(qscale) & 3u) != 0)
    return fail(LIME_ERR_INVALID_ARG, "bad_id_count and qscale must be 4-byte aligned");
  return ok();
}

static lime_status_t cand_score_impl(bool i8, lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                                     int32_t heads, const void* cache, const float* qscale,
                                     int64_t n_items, const void* links_pers, const int64_t* cand_ids,
                                     const int64_t* cand_offsets, int64_t total_M, void* out,
                                     int32_t* bad_id_count, void* stream) {
  const lime_status_t cs = check_score(i8, dtype, B, ell, d, heads, cache, qscale, n_items, links_pers,
                                       cand_ids, cand_offsets, total_M, out, bad_id_count);
  if (cs != LIME_OK) return cs;
  if (total_M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LIME_BF16) {
    const lime_status_t r =
        i8 ? try_cs_mfma<true>(ell, d, heads, cache, qscale, n_items, links_pers, cand_ids, cand_offsets, B,
                               total_M, out, bad_id_count, s)
           : try_cs_mfma<false>(ell, d, heads, cache, qscale, n_items, links_pers, cand_ids, cand_offsets, B,
                                total_M, out, bad_id_count, s);
    if (r != LIME_ERR_UNSUPPORTED) return r;
  }
  const int64_t n = total_M * d;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
#define LIME_CSG(T, I) \
  LIME_LAUNCH("gen::cand_score", (gen::cand_score<T, I>), grid, dim3(256), 0, s, cache, qscale, n_items, \
                     static_cast<const T*>(links_pers), cand_ids, cand_offsets, B, ell, d, heads, total_M, \
                     static_cast<T*>(out), bad_id_count)
  if (dtype == LIME_F32) {
    if (i8) LIME_CSG(float, true); else LIME_CSG(float, false);
  } else {
    if (i8) LIME_CSG(bf16_t, true); else LIME_CSG(bf16_t, false);
  }
#undef LIME_CSG
  LIME_CHECK_LAUNCH("candidate scoring");
  return ok();
}

lime_status_t lime_qk_cache_build(lime_dtype_t dtype, lime_phi_t phi, float scale,
                                  int64_t n_items, int32_t d, int32_t heads, int32_t ell,
                                  const void* items, const void* link_keys, void* cache,
                                  void* stream) {
  return qk_cache_impl(false, dtype, phi, scale, n_items, d, heads, ell, items, link_keys, cache, nullptr,
                       stream);
}

lime_status_t lime_qk_cache_build_i8(lime_dtype_t dtype, lime_phi_t phi, float scale,
                                     int64_t n_items, int32_t d, int32_t heads, int32_t ell,
                                     const void* items, const void* link_keys, int8_t* codes,
                                     float* qscale, void* stream) {
  return qk_cache_impl(true, dtype, phi, scale, n_items, d, heads, ell, items, link_keys, codes, qscale,
                       stream);
}

lime_status_t lime_cand_score(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                              int32_t heads, const void* cache, int64_t n_items,
                              const void* links_pers, const int64_t* cand_ids,
                              const int64_t* cand_offsets, int64_t total_M, void* out,
                              int32_t* bad_id_count, void* stream) {
  return cand_score_impl(false, dtype, B, ell, d, heads, cache, nullptr, n_items, links_pers, cand_ids,
                         cand_offsets, total_M, out, bad_id_count, stream);
}

lime_status_t lime_xor_fwd_score(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                                 int32_t ell, int32_t d, int32_t heads, int32_t layers, int32_t d_ff,
                                 const void* links_ctx, const void* hist, const int64_t* hist_offsets,
                                 int64_t total_N, int32_t max_N, const lime_layer_weights_t* w,
                                 void* links_pers, void* hist_out, void* workspace,
                                 size_t workspace_bytes, const void* cache, int64_t n_items,
                                 const int64_t* cand_ids, const int64_t* cand_offsets, int64_t total_M,
                                 void* out, int32_t* bad_id_count, void* stream) {
  // every argument of the scoring half is checked before anything launches
  const lime_status_t cs = check_score(false, dtype, B, ell, d, heads, cache, nullptr, n_items, links_pers,
                                       cand_ids, cand_offsets, total_M, out, bad_id_count);
  if (cs != LIME_OK) return cs;
  mfma::ScoreArgs sa;
  if (dtype == LIME_BF16 && total_M > 0) {
    sa.cache = static_cast<const bf16_t*>(cache);
    sa.n_items = n_items;
    sa.ids = cand_ids;
    sa.coff = cand_offsets;
    sa.total_M = total_M;
    sa.out = static_cast<bf16_t*>(out);
    sa.bad = bad_id_count;
  }
  bool scored = false;
  const lime_status_t xs = xor_fwd_impl(LIME_VARIANT_XOR, 0, dtype, phi, scale, B, ell, d, heads, layers, d_ff,
                                        links_ctx, hist, hist_offsets, total_N, max_N, w, links_pers, hist_out,
                                        workspace, workspace_bytes, stream, &sa, &scored);
  if (xs != LIME_OK || scored) return xs;
  return cand_score_impl(false, dtype, B, ell, d, heads, cache, nullptr, n_items, links_pers, cand_ids,
                         cand_offsets, total_M, out, bad_id_count, stream);
}

lime_status_t lime_cand_score_i8(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                                 int32_t heads, const int8_t* codes, const float* qscale,
                                 int64_t n_items, const void* links_pers, const int64_t* cand_ids,
                                 const int64_t* cand_offsets, int64_t total_M, void* out,
                                 int32_t* bad_id_count, void* stream) {
  return cand_score_impl(true, dtype, B, ell, d, heads, codes, qscale, n_items, links_pers, cand_ids,
                         cand_offsets, total_M, out, bad_id_count, stream);
}

lime_status_t lime_cand_score_uncached(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                                       int32_t ell, int32_t d, int32_t heads, const void* items,
                                       int64_t n_items, const void* link_keys, const void* links_pers,
                                       const int64_t* cand_ids, const int64_t* cand_offsets,
                                       int64_t total_M, void* out, int32_t* bad_id_count, void* stream) {
  if (dtype != LIME_F32 && dtype != LIME_BF16) return fail(LIME_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
  if (phi != LIME_PHI_SOFTMAX && phi != LIME_PHI_SILU_MEAN) return fail(LIME_ERR_INVALID_ARG, "bad phi %d", (int)phi);
  if (!std::isfinite(scale)) return fail(LIME_ERR_INVALID_ARG, "scale must be finite");
  if (B < 1 || ell < 1 || d < 1 || heads < 1 || n_items < 0 || total_M < 0)
    return fail(LIME_ERR_INVALID_ARG, "sizes must be positive");
  if (d % heads != 0) return fail(LIME_ERR_INVALID_ARG, "d (%d) must be a multiple of heads (%d)", d, heads);
  if (ell > 256) return fail(LIME_ERR_UNSUPPORTED, "ell > 256 unsupported (got %d)", ell);
  if (d % 8 != 0 || d > 1024) return fail(LIME_ERR_UNSUPPORTED, "d must be a multiple of 8 and <= 1024 (got %d)", d);
  if (heads > 65535) return fail(LIME_ERR_UNSUPPORTED, "too many heads");
  if (!link_keys || !links_pers || !cand_offsets) return fail(LIME_ERR_INVALID_ARG, "null pointer argument");
  if (total_M > 0 && (!cand_ids || !out)) return fail(LIME_ERR_INVALID_ARG, "null pointer argument");
  if (n_items > 0 && !items) return fail(LIME_ERR_INVALID_ARG, "items is null");
  if (!aligned16(items) || !aligned16(link_keys) || !aligned16(links_pers) || !aligned16(cand_ids) ||
      !aligned16(cand_offsets) || !aligned16(out))
    return fail(LIME_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(bad_id_count) & 3u) != 0)
    return fail(LIME_ERR_INVALID_ARG, "bad_id_count must be 4-byte aligned");
  if (total_M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LIME_BF16 && d == 32 * heads) {
    const int64_t ntiles = (total_M + 15) / 16;
#define LIME_UC(E, DD, HH)                                                                             \
    if (ell == E && d == DD && heads == HH) {                                                          \
      using UC = mfma::UcCfg<E, DD, HH>;                                                               \
      constexpr size_t lds = UC::lds_bytes;                                                            \
      /* about 16 waves per CU over all head groups */                                                 \
      const int64_t target_waves = static_cast<int64_t>(cu_count()) * 16 / UC::NHG;                    \
      int64_t tpw = (ntiles + target_waves - 1) / target_waves;                                        \
      if (tpw < 1) tpw = 1;                                                                            \
      const int64_t waves = (ntiles + tpw - 1) / tpw;                                                  \
      const dim3 grid(static_cast<unsigned>((waves + UC::NW - 1) / UC::NW), UC::NHG);                  \
      static const bool attr = hipFuncSetAttribute(                                                    \
          reinterpret_cast<const void*>(mfma::cand_score_uncached<E, DD, HH>),                         \
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) == hipSuccess;            \
      (void)attr;                                                                                      \
      LIME_LAUNCH("cand_score_uncached", (mfma::cand_score_uncached<E, DD, HH>), grid, dim3(UC::NT), lds, s,        \
                         static_cast<const bf16_t*>(items), n_items, static_cast<const bf16_t*>(link_keys), \
                         static_cast<const bf16_t*>(links_pers), cand_ids, cand_offsets, B, total_M,   \
                         static_cast<bf16_t*>(out), bad_id_count, scale, static_cast<int>(phi), tpw);  \
      LIME_CHECK_LAUNCH("uncached scoring (mfma)");                                                    \
      return ok();                                                                                     \
    }
    LIME_UC(32, 64, 2) LIME_UC(32, 128, 4) LIME_UC(64, 128, 4) LIME_UC(32, 256, 8) LIME_UC(64, 256, 8)
#undef LIME_UC
  }
  const dim3 grid(static_cast<unsigned>((total_M + 63) / 64), heads);
  const size_t lds = 64 * static_cast<size_t>(ell) * 4;
  if (dtype == LIME_F32)
    LIME_LAUNCH("gen::cand_score_uncached", gen::cand_score_uncached<float>, grid, dim3(64), lds, s, static_cast<const float*>(items),
                       n_items, static_cast<const float*>(link_keys), static_cast<const float*>(links_pers),
                       cand_ids, cand_offsets, B, ell, d, heads, total_M, static_cast<float*>(out), bad_id_count,
                       scale, static_cast<int>(phi));
  else
    LIME_LAUNCH("gen::cand_score_uncached", gen::cand_score_uncached<bf16_t>, grid, dim3(64), lds, s, static_cast<const bf16_t*>(items),
                       n_items, static_cast<const bf16_t*>(link_keys), static_cast<const bf16_t*>(links_pers),
                       cand_ids, cand_offsets, B, ell, d, heads, total_M, static_cast<bf16_t*>(out), bad_id_count,
                       scale, static_cast<int>(phi));
  LIME_CHECK_LAUNCH("uncached scoring");
  return ok();
}

}  // extern "C"
