// C-ABI of the fused block (include/coda.h): argument checks, workspace
// layout and the launch sequence of each entry point.  Every check runs
// before the first HIP call, so a rejected call touches neither the device
// nor the stream.
#include "../../include/coda.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "launch.hpp"

namespace {

using coda::GemmArgs;

// Size limits.  The GEMM loaders reach an operand through buffer windows of
// at most 2 GiB: a K-contiguous operand's window holds the tile's 256 rows, an
// MN-contiguous operand's window one K step (at most 64 rows), so a tensor may
// be far larger than 2 GiB as long as its rows are not too long.  Every
// contiguous row length (K, d, N, F, 2F, V) is at most 2^21 elements, the row
// count M at most 2^23 (M is the contiguous index of y*gamma stored
// transposed), and no tensor exceeds 1 TiB.
constexpr uint64_t kMaxTensorBytes = 1ull << 40;
constexpr int64_t kMaxRowLen = (int64_t)1 << 21;
constexpr int64_t kMaxRows = (int64_t)1 << 23;
static_assert(coda::kNoAllocScratchBytes == CODA_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
constexpr size_t kAlign = 256;

size_t esize(coda_dtype t) { return t == CODA_BF16 ? 2 : 4; }
bool dtype_ok(int t) { return t == CODA_F32 || t == CODA_BF16; }
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// a row length (K, d, N, F, V); the token count M goes through rows_ok
bool dim_ok(coda_dtype t, int64_t v) {
  const int64_t q = t == CODA_BF16 ? 8 : 4;
  return v >= q && v % q == 0 && v <= kMaxRowLen;
}
bool rows_ok(coda_dtype t, int64_t v) {
  const int64_t q = t == CODA_BF16 ? 8 : 4;
  return v >= q && v % q == 0 && v <= kMaxRows;
}
bool bytes_ok(coda_dtype t, int64_t a, int64_t b) {
  return (uint64_t)a * (uint64_t)b * esize(t) <= kMaxTensorBytes;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, uint64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Outputs may not overlap inputs, other outputs or the workspace.
template <int NI, int NO>
bool alias_free(const Range (&in)[NI], const Range (&out)[NO]) {
  for (int o = 0; o < NO; ++o) {
    if (out[o].hi == out[o].lo) continue;
    for (int i = 0; i < NI; ++i)
      if (in[i].hi != in[i].lo && overlap(out[o], in[i])) return false;
    for (int p = o + 1; p < NO; ++p)
      if (out[p].hi != out[p].lo && overlap(out[o], out[p])) return false;
  }
  return true;
}

coda_status hip_status(hipError_t e) { return e == hipSuccess ? CODA_OK : CODA_ERR_HIP; }

// ------------------------------------------------------------- tracing
struct TraceRec {
  const char* name;
  double flops, bytes;
};
struct TraceState {
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;   // two per launch
  std::vector<TraceRec> rec;
};
TraceState g_trace;

// Enqueue one kernel through `f`, bracketed by trace events when tracing is on.
template <class Fn>
hipError_t traced(const char* name, double flops, double bytes, hipStream_t s, Fn f) {
  int i = -1;
  if (g_trace.on && g_trace.n < g_trace.cap) {
    i = g_trace.n++;
    g_trace.rec[i] = {name, flops, bytes};
    hipEventRecord(g_trace.ev[2 * i], s);
  }
  const hipError_t e = f();
  if (i >= 0) hipEventRecord(g_trace.ev[2 * i + 1], s);
  return e;
}

double gemm_flops(int64_t M, int64_t N, int64_t K) { return 2.0 * (double)M * (double)N * (double)K; }

// ------------------------------------------------------------- workspaces
// Forward workspace: P [M, Tn] fp32 partial sums of squares, yg = y * gamma
// (the second GEMM's A operand, written by the first GEMM's epilogue): bf16
// stored transposed, [d, M], so that both operands of the second GEMM are
// MN-contiguous; fp32 stored [M, d].
struct FwdWs {
  size_t P, yg, total;
  int Tn;
};
FwdWs fwd_ws(coda_dtype t, int64_t M, int64_t d, int64_t N) {
  (void)N;
  FwdWs w;
  w.Tn = (int)cdiv(d, t == CODA_BF16 ? coda::kTileN : coda::kTileF32);
  w.P = 0;
  w.yg = round_up((size_t)M * w.Tn * 4);
  w.total = w.yg + round_up((size_t)M * d * esize(t));
  return w;
}

struct BwdWs {
  size_t n, S, G, c, total;
  int Tn, Tm;
};
BwdWs bwd_ws(int64_t M, int64_t d) {
  BwdWs w;
  w.Tn = (int)cdiv(d, coda::kTileN);
  w.Tm = (int)cdiv(M, coda::kTileM);
  w.n = 0;
  w.S = round_up((size_t)M * d * 2);
  w.G = w.S + round_up((size_t)M * w.Tn * 4);
  w.c = w.G + round_up((size_t)w.Tm * d * 4);
  w.total = w.c + round_up((size_t)M * 4);
  return w;
}

GemmArgs gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, uint64_t A_elems,
              const void* B, int64_t ldb, uint64_t B_elems, void* C, int64_t ldc) {
  GemmArgs g{};
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.A = A;
  g.lda = lda;
  g.A_total = A_elems * 2;
  g.A_bytes = (uint32_t)std::min<uint64_t>(g.A_total, 0x7FFFFFF0ull);
  g.B = B;
  g.ldb = ldb;
  g.B_total = B_elems * 2;
  g.B_bytes = (uint32_t)std::min<uint64_t>(g.B_total, 0x7FFFFFF0ull);
  g.C = C;
  g.ldc = ldc;
  return g;
}

// K1: y = X W1 + R; the epilogue stores y, yg = y * gamma (bf16: transposed,
// [d, M]) and the per-tile partial sums of squares P.
hipError_t launch_k1(bool bf, int64_t M, int64_t K, int64_t d, const void* X, const void* W1,
                     const void* R, const void* gamma, void* y, const FwdWs& ws, float* P,
                     void* yg, hipStream_t s, bool yg_trans = true) {
  const double eb = bf ? 2.0 : 4.0;
  GemmArgs g1 = gemm(M, d, K, X, K, M * K, W1, d, K * d, y, d);
  g1.E = R;
  g1.lde = d;
  g1.part_row = P;
  g1.ld_part_row = ws.Tn;
  g1.C2 = yg;
  g1.ldc2 = bf && yg_trans ? M : d;
  g1.c2_trans = bf && yg_trans ? 1 : 0;
  g1.vcol = gamma;
  const double k1_bytes = (M * K + K * d + 3.0 * M * d + d) * eb + M * ws.Tn * 4.0;
  return traced("k1_gemm_resid_sumsq", gemm_flops(M, d, K), k1_bytes, s, [&] {
    return bf ? coda::launch_gemm_bf16(g1, true, false, coda::EPI_RESID_SUMSQ, s)
              : coda::launch_gemm_f32(g1, coda::EPI_RESID_SUMSQ, s);
  });
}

// The RMS-normalised block's backward after its second GEMM, given that
// GEMM's output gradient dz [M, N] and weight W2 [d, N]: B1 (dh = dz W2^T and
// the dn / n / s / dgamma epilogue), R2, E2 (dy, plus dy_in when not NULL),
// B2 (dW2), B3 (dX), B4 (dW1).  `nm` names the six launches for tracing.
hipError_t launch_norm_bwd(int64_t M, int64_t K, int64_t d, int64_t N, const void* X,
                           const void* W1, const void* gamma, const void* W2, const void* y,
                           const float* r, const void* dz, const void* dy_in, void* dX, void* dW1,
                           void* dR, void* dW2, float* dgamma, const BwdWs& ws, char* wsb,
                           const char* const (&nm)[6], hipStream_t s) {
  void* n = wsb + ws.n;
  float* S = (float*)(wsb + ws.S);
  float* G = (float*)(wsb + ws.G);
  float* c = (float*)(wsb + ws.c);
  hipError_t err;

  // B1: dh = dz W2^T; epilogue -> dn (into dR), row partials S, column partials G
  GemmArgs b1 = gemm(M, d, N, dz, N, M * N, W2, N, d * N, dR, d);
  b1.E = y;
  b1.lde = d;
  b1.vrow = r;
  b1.vcol = gamma;
  b1.part_row = S;
  b1.ld_part_row = ws.Tn;
  b1.part_col = G;
  b1.ld_part_col = d;
  b1.C2 = n;                      // n = r * y, the A operand of the dW2 GEMM
  b1.ldc2 = d;
  const double md = 2.0 * M * d, dn2 = 2.0 * d * N, mn = 2.0 * M * N, mk = 2.0 * M * K, kd = 2.0 * K * d;
  if ((err = traced(nm[0], gemm_flops(M, d, N),
                    mn + dn2 + 3.0 * md + M * ws.Tn * 4.0 + ws.Tm * d * 4.0 + M * 4.0 + 2.0 * d, s,
                    [&] { return coda::launch_gemm_bf16(b1, true, true, coda::EPI_DN, s); })) !=
      hipSuccess)
    return err;
  // R2: c = r^3 s / d, dgamma
  if ((err = traced(nm[1], 0.0, M * ws.Tn * 4.0 + ws.Tm * d * 4.0 + 8.0 * M + 4.0 * d, s, [&] {
         return coda::launch_bwd_reduce(S, ws.Tn, ws.Tn, r, M, d, G, ws.Tm, c, dgamma, s);
       })) != hipSuccess)
    return err;
  // E2: dR = r dn - c y (+ dy_in), in place
  if ((err = traced(nm[2], 0.0, (dy_in ? 4.0 : 3.0) * md + 8.0 * M, s,
                    [&] { return coda::launch_dy(dR, y, r, c, dy_in, M, d, s); })) != hipSuccess)
    return err;
  // B2: dW2 = diag(gamma) n^T dz
  GemmArgs b2 = gemm(d, N, M, n, d, M * d, dz, N, M * N, dW2, N);
  b2.vcol = gamma;
  if ((err = traced(nm[3], gemm_flops(d, N, M), md + mn + dn2 + 2.0 * d, s, [&] {
         return coda::launch_gemm_bf16(b2, false, false, coda::EPI_ROWSCALE, s);
       })) != hipSuccess)
    return err;
  // B3: dX = dy W1^T
  GemmArgs b3 = gemm(M, K, d, dR, d, M * d, W1, d, K * d, dX, K);
  if ((err = traced(nm[4], gemm_flops(M, K, d), md + kd + mk, s, [&] {
         return coda::launch_gemm_bf16(b3, true, true, coda::EPI_STORE, s);
       })) != hipSuccess)
    return err;
  // B4: dW1 = X^T dy
  GemmArgs b4 = gemm(K, d, M, X, K, M * K, dR, d, M * d, dW1, d);
  return traced(nm[5], gemm_flops(K, d, M), mk + md + kd, s, [&] {
    return coda::launch_gemm_bf16(b4, false, false, coda::EPI_STORE, s);
  });
}

// ------------------------------------------------------------- MXFP8
bool mx_dim_ok(int64_t v, int64_t q) { return v >= q && v % q == 0 && v <= kMaxRowLen; }
bool mx_rows_ok(int64_t v, int64_t q) { return v >= q && v % q == 0 && v <= kMaxRows; }
bool fits(int64_t a, int64_t b, int64_t e) { return (uint64_t)a * (uint64_t)b * (uint64_t)e <= kMaxTensorBytes; }
// MXFP8 scales are read through one buffer of at most 2 GiB
bool scales_fit(int64_t rows, int64_t cols) { return (uint64_t)rows * (uint64_t)(cols / 32) <= 0x7FFFFFF0ull; }

struct Mx8Ws {
  size_t P, q, qs, total;
  int Tn;
};
Mx8Ws mx8_ws(int64_t M, int64_t d) {
  Mx8Ws w;
  w.Tn = (int)cdiv(d, coda::kTileN);
  w.P = 0;
  w.q = round_up((size_t)M * w.Tn * 4);
  w.qs = w.q + round_up((size_t)M * d);
  w.total = w.qs + round_up((size_t)M * (d / 32));
  return w;
}

// An MXFP8 GEMM C = A B with A [M][K] and B^T [N][K] (codes) and their scales.
GemmArgs gemm_mx8(int64_t M, int64_t N, int64_t K, const void* Aq, const void* As, const void* Bq,
                  const void* Bs, void* C, int64_t ldc) {
  GemmArgs g{};
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.A = Aq;
  g.lda = K;
  g.A_total = (uint64_t)(M * K);
  g.A_bytes = (uint32_t)std::min<uint64_t>(g.A_total, 0x7FFFFFF0ull);
  g.B = Bq;
  g.ldb = K;
  g.B_total = (uint64_t)(N * K);
  g.B_bytes = (uint32_t)std::min<uint64_t>(g.B_total, 0x7FFFFFF0ull);
  g.sA = (const uint8_t*)As;
  g.sB = (const uint8_t*)Bs;
  g.sA_bytes = (uint32_t)(M * (K / 32));
  g.sB_bytes = (uint32_t)(N * (K / 32));
  g.C = C;
  g.ldc = ldc;
  return g;
}

}  // namespace

extern "C" {

const char* coda_status_str(coda_status s) {
  switch (s) {
    case CODA_OK: return "CODA_OK";
    case CODA_ERR_NULL: return "CODA_ERR_NULL: a required pointer is NULL";
    case CODA_ERR_SHAPE: return "CODA_ERR_SHAPE: a size is out of range or not a multiple of 8 (bf16) / 4 (f32)";
    case CODA_ERR_ALIGN: return "CODA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case CODA_ERR_ALIAS: return "CODA_ERR_ALIAS: an output overlaps an input, another output or the workspace";
    case CODA_ERR_DTYPE: return "CODA_ERR_DTYPE: unknown dtype";
    case CODA_ERR_EPS: return "CODA_ERR_EPS: eps must be finite and > 0";
    case CODA_ERR_WORKSPACE: return "CODA_ERR_WORKSPACE: workspace missing or too small";
    case CODA_ERR_UNSUPPORTED: return "CODA_ERR_UNSUPPORTED: not implemented for this dtype";
    case CODA_ERR_HIP: return "CODA_ERR_HIP: a HIP call or kernel launch failed";
  }
  return "CODA_ERR_UNKNOWN";
}

const char* coda_version(void) { return "coda-mi355x 0.1.0 gfx950"; }

size_t coda_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N) {
  (void)K;
  if (!dtype_ok(dtype) || M < 1 || d < 1 || N < 1) return 0;
  return fwd_ws(dtype, M, d, N).total;
}

}  // extern "C"

namespace {

// coda_fwd's checks of everything but the workspace.
coda_status fwd_check(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N, float eps,
                      const void* X, const void* W1, const void* R, const void* gamma,
                      const void* W2, void* y, float* r, void* z) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W1 || !R || !gamma || !W2 || !y || !r || !z) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, K) || !dim_ok(dtype, d) || !dim_ok(dtype, N))
    return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, K) || !bytes_ok(dtype, K, d) || !bytes_ok(dtype, M, d) ||
      !bytes_ok(dtype, d, N) || !bytes_ok(dtype, M, N))
    return CODA_ERR_SHAPE;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return CODA_ERR_EPS;
  for (const void* p : {X, W1, R, gamma, W2, (const void*)y, (const void*)r, (const void*)z})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  return CODA_OK;
}

// Outputs against inputs, each other and the workspace.
bool fwd_alias_free(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N, const void* X,
                    const void* W1, const void* R, const void* gamma, const void* W2, void* y,
                    float* r, void* z, const void* workspace, size_t ws_bytes) {
  const size_t e = esize(dtype);
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(R, M * d * e), rng(gamma, d * e),
                      rng(W2, d * N * e)};
  const Range out[] = {rng(y, M * d * e), rng(r, M * 4), rng(z, M * N * e), rng(workspace, ws_bytes)};
  return alias_free(in, out);
}

// The forward's launches, with the partial sums and y*gamma in `wsb`.
coda_status fwd_launch(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N, float eps,
                       const void* X, const void* W1, const void* R, const void* gamma,
                       const void* W2, void* y, float* r, void* z, const FwdWs& ws, char* wsb,
                       hipStream_t s) {
  float* P = (float*)(wsb + ws.P);
  void* yg = wsb + ws.yg;
  hipError_t err;
  const double eb = (double)esize(dtype);

  const bool bf = dtype == CODA_BF16;
  // y*gamma layout: stored transposed ([d, M]) so that K2 runs with both
  // operands MN-contiguous, unless K2's operands are small enough to stay in
  // the MALL (at most 128 MiB), where the row-major store (cheaper in K1's
  // epilogue) and a K-contiguous A on 64-k steps are faster (measured: the
  // LLaMA-1B-shaped forward 2.4% faster that way, the LLaMA-7B-shaped one
  // 0.9% slower)
  const bool yg_t = ((double)M + (double)N) * (double)d * 2.0 > 128.0 * 1048576.0;
  if ((err = launch_k1(bf, M, K, d, X, W1, R, gamma, y, ws, P, yg, s, yg_t)) != hipSuccess)
    return hip_status(err);
  // K2: z = diag(r) (yg W2); bf16 reads a transposed yg [d, M] as an
  // MN-contiguous A
  GemmArgs g2 = gemm(M, N, d, yg, bf && yg_t ? M : d, M * d, W2, N, d * N, z, N);
  const double k2_bytes = (M * d + d * N + M * N) * eb + M * ws.Tn * 4.0 + M * 4.0;
  if (bf) {
    // r is formed in K2's epilogue from the partial sums (and written by the
    // tiles of the first column)
    g2.part_row = P;
    g2.ld_part_row = ws.Tn;
    g2.nparts = ws.Tn;
    g2.inv_d = 1.0f / (float)d;
    g2.eps = eps;
    g2.r_out = r;
    return hip_status(traced("k2_gemm_rsqrt_rowscale", gemm_flops(M, N, d), k2_bytes, s, [&] {
      return coda::launch_gemm_bf16(g2, !yg_t, false, coda::EPI_RSQRT_SCALE, s);
    }));
  }
  if ((err = traced("r1_row_rsqrt", 0.0, M * ws.Tn * 4.0 + M * 4.0, s, [&] {
         return coda::launch_row_rsqrt(P, ws.Tn, ws.Tn, M, d, eps, r, s);
       })) != hipSuccess)
    return hip_status(err);
  g2.vrow = r;
  return hip_status(traced("k2_gemm_rowscale", gemm_flops(M, N, d), k2_bytes, s, [&] {
    return coda::launch_gemm_f32(g2, coda::EPI_ROWSCALE, s);
  }));
}

}  // namespace

extern "C" {

coda_status coda_fwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N, float eps,
                     const void* X, const void* W1, const void* R, const void* gamma,
                     const void* W2, void* y, float* r, void* z, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const coda_status st = fwd_check(dtype, M, K, d, N, eps, X, W1, R, gamma, W2, y, r, z);
  if (st != CODA_OK) return st;
  const FwdWs ws = fwd_ws(dtype, M, d, N);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  if (!fwd_alias_free(dtype, M, K, d, N, X, W1, R, gamma, W2, y, r, z, workspace, ws.total))
    return CODA_ERR_ALIAS;
  return fwd_launch(dtype, M, K, d, N, eps, X, W1, R, gamma, W2, y, r, z, ws, (char*)workspace,
                    (hipStream_t)stream);
}

coda_status coda_fwd_noalloc(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N,
                             float eps, const void* X, const void* W1, const void* R,
                             const void* gamma, const void* W2, void* y, float* r, void* z,
                             void* stream) {
  const coda_status st = fwd_check(dtype, M, K, d, N, eps, X, W1, R, gamma, W2, y, r, z);
  if (st != CODA_OK) return st;
  const FwdWs ws = fwd_ws(dtype, M, d, N);
  if (ws.total > coda::kNoAllocScratchBytes) return CODA_ERR_WORKSPACE;
  // the scratch is the library's own array, which no caller buffer can overlap
  if (!fwd_alias_free(dtype, M, K, d, N, X, W1, R, gamma, W2, y, r, z, nullptr, 0))
    return CODA_ERR_ALIAS;
  void* scratch = nullptr;
  if (coda::noalloc_scratch(&scratch) != hipSuccess) return CODA_ERR_HIP;
  return fwd_launch(dtype, M, K, d, N, eps, X, W1, R, gamma, W2, y, r, z, ws, (char*)scratch,
                    (hipStream_t)stream);
}

size_t coda_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N) {
  (void)K;
  (void)N;
  if (dtype != CODA_BF16 || M < 1 || d < 1) return 0;
  return bwd_ws(M, d).total;
}

coda_status coda_bwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N,
                     const void* X, const void* W1, const void* gamma, const void* W2,
                     const void* y, const float* r, const void* dz, void* dX, void* dW1,
                     void* dR, void* dW2, float* dgamma, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W1 || !gamma || !W2 || !y || !r || !dz || !dX || !dW1 || !dR || !dW2 || !dgamma)
    return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, K) || !dim_ok(dtype, d) || !dim_ok(dtype, N))
    return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, K) || !bytes_ok(dtype, K, d) || !bytes_ok(dtype, M, d) ||
      !bytes_ok(dtype, d, N) || !bytes_ok(dtype, M, N))
    return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W1, gamma, W2, y, (const void*)r, dz, (const void*)dX,
                        (const void*)dW1, (const void*)dR, (const void*)dW2, (const void*)dgamma})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const BwdWs ws = bwd_ws(M, d);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(gamma, d * e), rng(W2, d * N * e),
                      rng(y, M * d * e), rng(r, M * 4), rng(dz, M * N * e)};
  const Range out[] = {rng(dX, M * K * e), rng(dW1, K * d * e), rng(dR, M * d * e),
                       rng(dW2, d * N * e), rng(dgamma, d * 4), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  static const char* const names[6] = {"b1_gemm_dh_epilogue", "r2_bwd_reduce", "e2_dy",
                                       "b2_gemm_dW2", "b3_gemm_dX", "b4_gemm_dW1"};
  return hip_status(launch_norm_bwd(M, K, d, N, X, W1, gamma, W2, y, r, dz, nullptr, dX, dW1, dR,
                                    dW2, dgamma, ws, (char*)workspace, names,
                                    (hipStream_t)stream));
}

size_t coda_swiglu_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t F) {
  (void)dtype;
  (void)M;
  (void)d;
  (void)F;
  return 0;
}

coda_status coda_swiglu_fwd(coda_dtype dtype, int64_t M, int64_t d, int64_t F, const void* X,
                            const void* W, const void* Wd, void* gu, void* a, void* z,
                            void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W || !Wd || !gu || !a || !z) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, d) || !dim_ok(dtype, F) || !dim_ok(dtype, 2 * F))
    return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, d) || !bytes_ok(dtype, d, 2 * F) || !bytes_ok(dtype, F, d) ||
      !bytes_ok(dtype, M, 2 * F))
    return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W, Wd, (const void*)gu, (const void*)a, (const void*)z})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * d * e), rng(W, d * 2 * F * e), rng(Wd, F * d * e)};
  const Range out[] = {rng(gu, M * 2 * F * e), rng(a, M * F * e), rng(z, M * d * e)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  hipError_t err;
  GemmArgs s1 = gemm(M, F, d, X, d, M * d, W, 2 * F, d * 2 * F, gu, 2 * F);
  s1.C2 = a;
  s1.ldc2 = F;
  s1.F = (int)F;
  const double Md = 2.0 * M * d, dF2 = 4.0 * d * F, MF = 2.0 * M * F, Fd = 2.0 * F * d;
  if ((err = traced("s1_gemm_gateup_swiglu", gemm_flops(M, 2 * F, d), Md + dF2 + 3.0 * MF, s, [&] {
         return coda::launch_gemm_bf16(s1, true, false, coda::EPI_SWIGLU, s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs s2 = gemm(M, d, F, a, F, M * F, Wd, d, F * d, z, d);
  return hip_status(traced("s2_gemm_down", gemm_flops(M, d, F), MF + Fd + Md, s, [&] {
    return coda::launch_gemm_bf16(s2, true, false, coda::EPI_STORE, s);
  }));
}

size_t coda_swiglu_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t F) {
  (void)d;
  if (dtype != CODA_BF16 || M < 1 || F < 1) return 0;
  return round_up((size_t)M * 2 * F * 2);
}

coda_status coda_swiglu_bwd(coda_dtype dtype, int64_t M, int64_t d, int64_t F, const void* X,
                            const void* W, const void* Wd, const void* gu, const void* a,
                            const void* dz, void* dX, void* dW, void* dWd, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W || !Wd || !gu || !a || !dz || !dX || !dW || !dWd) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, d) || !dim_ok(dtype, F) || !dim_ok(dtype, 2 * F))
    return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, d) || !bytes_ok(dtype, d, 2 * F) || !bytes_ok(dtype, F, d) ||
      !bytes_ok(dtype, M, 2 * F))
    return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W, Wd, gu, a, dz, (const void*)dX, (const void*)dW, (const void*)dWd})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const size_t need = coda_swiglu_bwd_workspace_bytes(dtype, M, d, F);
  if (!workspace || workspace_bytes < need) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * d * e), rng(W, d * 2 * F * e), rng(Wd, F * d * e),
                      rng(gu, M * 2 * F * e), rng(a, M * F * e), rng(dz, M * d * e)};
  const Range out[] = {rng(dX, M * d * e), rng(dW, d * 2 * F * e), rng(dWd, F * d * e),
                       rng(workspace, need)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  void* dgu = workspace;
  hipError_t err;
  // S3: da = dz Wd^T; epilogue -> dgu from the saved gu
  GemmArgs s3 = gemm(M, F, d, dz, d, M * d, Wd, d, F * d, dgu, 2 * F);
  s3.E = gu;
  s3.lde = 2 * F;
  s3.F = (int)F;
  const double Md = 2.0 * M * d, dF2 = 4.0 * d * F, MF = 2.0 * M * F, Fd = 2.0 * F * d;
  if ((err = traced("s3_gemm_da_swiglu_bwd", gemm_flops(M, F, d), Md + Fd + 4.0 * MF, s, [&] {
         return coda::launch_gemm_bf16(s3, true, true, coda::EPI_SWIGLU_BWD, s);
       })) != hipSuccess)
    return hip_status(err);
  // S4: dWd = a^T dz
  GemmArgs s4 = gemm(F, d, M, a, F, M * F, dz, d, M * d, dWd, d);
  if ((err = traced("s4_gemm_dWd", gemm_flops(F, d, M), MF + Md + Fd, s, [&] {
         return coda::launch_gemm_bf16(s4, false, false, coda::EPI_STORE, s);
       })) != hipSuccess)
    return hip_status(err);
  // S5: dX = dgu W^T
  GemmArgs s5 = gemm(M, d, 2 * F, dgu, 2 * F, M * 2 * F, W, 2 * F, d * 2 * F, dX, d);
  if ((err = traced("s5_gemm_dX", gemm_flops(M, d, 2 * F), 2.0 * MF + dF2 + Md, s, [&] {
         return coda::launch_gemm_bf16(s5, true, true, coda::EPI_STORE, s);
       })) != hipSuccess)
    return hip_status(err);
  // S6: dW = X^T dgu
  GemmArgs s6 = gemm(d, 2 * F, M, X, d, M * d, dgu, 2 * F, M * 2 * F, dW, 2 * F);
  return hip_status(traced("s6_gemm_dW", gemm_flops(d, 2 * F, M), Md + 2.0 * MF + dF2, s, [&] {
    return coda::launch_gemm_bf16(s6, false, false, coda::EPI_STORE, s);
  }));
}

coda_status coda_trace_start(int capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return CODA_ERR_SHAPE;
  coda_trace_stop();
  g_trace.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& e : g_trace.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      coda_trace_stop();
      return CODA_ERR_HIP;
    }
  }
  g_trace.rec.assign(capacity, TraceRec{nullptr, 0.0, 0.0});
  g_trace.cap = capacity;
  g_trace.n = 0;
  g_trace.on = true;
  return CODA_OK;
}

int coda_trace_count(void) { return g_trace.n; }

coda_status coda_trace_get(int index, const char** name, float* ms, double* flops, double* bytes) {
  if (index < 0 || index >= g_trace.n) return CODA_ERR_SHAPE;
  if (!name || !ms || !flops || !bytes) return CODA_ERR_NULL;
  if (hipEventSynchronize(g_trace.ev[2 * index + 1]) != hipSuccess) return CODA_ERR_HIP;
  if (hipEventElapsedTime(ms, g_trace.ev[2 * index], g_trace.ev[2 * index + 1]) != hipSuccess)
    return CODA_ERR_HIP;
  *name = g_trace.rec[index].name;
  *flops = g_trace.rec[index].flops;
  *bytes = g_trace.rec[index].bytes;
  return CODA_OK;
}

coda_status coda_trace_stop(void) {
  coda_status st = CODA_OK;
  for (auto& e : g_trace.ev)
    if (e && hipEventDestroy(e) != hipSuccess) st = CODA_ERR_HIP;
  g_trace.ev.clear();
  g_trace.rec.clear();
  g_trace.cap = g_trace.n = 0;
  g_trace.on = false;
  return st;
}

// ------------------------------------------------------- MLP sub-layer chain

size_t coda_mlp_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F) {
  (void)K;
  (void)F;
  if (dtype != CODA_BF16 || M < 1 || d < 1) return 0;
  return fwd_ws(dtype, M, d, 0).total;
}

coda_status coda_mlp_fwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F, float eps,
                         const void* X, const void* W1, const void* R, const void* gamma,
                         const void* W, const void* Wd, void* y, float* r, void* gu, void* a,
                         void* z, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W1 || !R || !gamma || !W || !Wd || !y || !r || !gu || !a || !z) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, K) || !dim_ok(dtype, d) || !dim_ok(dtype, F) ||
      !dim_ok(dtype, 2 * F))
    return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, K) || !bytes_ok(dtype, K, d) || !bytes_ok(dtype, M, d) ||
      !bytes_ok(dtype, d, 2 * F) || !bytes_ok(dtype, F, d) || !bytes_ok(dtype, M, 2 * F))
    return CODA_ERR_SHAPE;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return CODA_ERR_EPS;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W1, R, gamma, W, Wd, (const void*)y, (const void*)r, (const void*)gu,
                        (const void*)a, (const void*)z})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const FwdWs ws = fwd_ws(dtype, M, d, 0);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(R, M * d * e), rng(gamma, d * e),
                      rng(W, d * 2 * F * e), rng(Wd, F * d * e)};
  const Range out[] = {rng(y, M * d * e), rng(r, M * 4), rng(gu, M * 2 * F * e),
                       rng(a, M * F * e), rng(z, M * d * e), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  float* P = (float*)(wsb + ws.P);
  void* yg = wsb + ws.yg;
  hipError_t err;
  if ((err = launch_k1(true, M, K, d, X, W1, R, gamma, y, ws, P, yg, s)) != hipSuccess)
    return hip_status(err);
  // M1: [g | u] = diag(r) (yg W); epilogue: r from the partial sums (tiles of
  // the first column store it), both halves scaled by r, gu and a = silu(g) u
  GemmArgs m1 = gemm(M, F, d, yg, M, M * d, W, 2 * F, d * 2 * F, gu, 2 * F);
  m1.C2 = a;
  m1.ldc2 = F;
  m1.F = (int)F;
  m1.part_row = P;
  m1.ld_part_row = ws.Tn;
  m1.nparts = ws.Tn;
  m1.inv_d = 1.0f / (float)d;
  m1.eps = eps;
  m1.r_out = r;
  const double Md = 2.0 * M * d, dF2 = 4.0 * d * F, MF = 2.0 * M * F, Fd = 2.0 * F * d;
  if ((err = traced("m1_gemm_gateup_rsqrt_swiglu", gemm_flops(M, 2 * F, d),
                    Md + dF2 + 3.0 * MF + M * ws.Tn * 4.0 + M * 4.0, s, [&] {
                      return coda::launch_gemm_bf16(m1, false, false, coda::EPI_RSQRT_SWIGLU, s);
                    })) != hipSuccess)
    return hip_status(err);
  // M2: z = a Wd
  GemmArgs m2 = gemm(M, d, F, a, F, M * F, Wd, d, F * d, z, d);
  return hip_status(traced("m2_gemm_down", gemm_flops(M, d, F), MF + Fd + Md, s, [&] {
    return coda::launch_gemm_bf16(m2, true, false, coda::EPI_STORE, s);
  }));
}

size_t coda_mlp_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F) {
  (void)K;
  if (dtype != CODA_BF16 || M < 1 || d < 1 || F < 1) return 0;
  return round_up((size_t)M * 2 * F * 2) + bwd_ws(M, d).total;
}

coda_status coda_mlp_bwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F,
                         const void* X, const void* W1, const void* gamma, const void* W,
                         const void* Wd, const void* y, const float* r, const void* gu,
                         const void* a, const void* dz, const void* dy_in, void* dX, void* dW1,
                         void* dR, void* dW, void* dWd, float* dgamma, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W1 || !gamma || !W || !Wd || !y || !r || !gu || !a || !dz || !dX || !dW1 || !dR ||
      !dW || !dWd || !dgamma)
    return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, K) || !dim_ok(dtype, d) || !dim_ok(dtype, F) ||
      !dim_ok(dtype, 2 * F))
    return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, K) || !bytes_ok(dtype, K, d) || !bytes_ok(dtype, M, d) ||
      !bytes_ok(dtype, d, 2 * F) || !bytes_ok(dtype, F, d) || !bytes_ok(dtype, M, 2 * F))
    return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W1, gamma, W, Wd, y, (const void*)r, gu, a, dz, (const void*)dX,
                        (const void*)dW1, (const void*)dR, (const void*)dW, (const void*)dWd,
                        (const void*)dgamma})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  if (dy_in && !aligned16(dy_in)) return CODA_ERR_ALIGN;
  const size_t dgu_bytes = round_up((size_t)M * 2 * F * 2);
  const BwdWs ws = bwd_ws(M, d);
  if (!workspace || workspace_bytes < dgu_bytes + ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(gamma, d * e),
                      rng(W, d * 2 * F * e), rng(Wd, F * d * e), rng(y, M * d * e), rng(r, M * 4),
                      rng(gu, M * 2 * F * e), rng(a, M * F * e), rng(dz, M * d * e),
                      rng(dy_in, dy_in ? M * d * e : 0)};
  const Range out[] = {rng(dX, M * K * e), rng(dW1, K * d * e), rng(dR, M * d * e),
                       rng(dW, d * 2 * F * e), rng(dWd, F * d * e), rng(dgamma, d * 4),
                       rng(workspace, dgu_bytes + ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  void* dgu = wsb;
  hipError_t err;
  // M3: da = dz Wd^T; epilogue -> dgu = [dg | du] from the saved gu
  GemmArgs m3 = gemm(M, F, d, dz, d, M * d, Wd, d, F * d, dgu, 2 * F);
  m3.E = gu;
  m3.lde = 2 * F;
  m3.F = (int)F;
  const double Md = 2.0 * M * d, MF = 2.0 * M * F, Fd = 2.0 * F * d;
  if ((err = traced("m3_gemm_da_swiglu_bwd", gemm_flops(M, F, d), Md + Fd + 4.0 * MF, s, [&] {
         return coda::launch_gemm_bf16(m3, true, true, coda::EPI_SWIGLU_BWD, s);
       })) != hipSuccess)
    return hip_status(err);
  // M4: dWd = a^T dz
  GemmArgs m4 = gemm(F, d, M, a, F, M * F, dz, d, M * d, dWd, d);
  if ((err = traced("m4_gemm_dWd", gemm_flops(F, d, M), MF + Md + Fd, s, [&] {
         return coda::launch_gemm_bf16(m4, false, false, coda::EPI_STORE, s);
       })) != hipSuccess)
    return hip_status(err);
  // the normalised block's backward with [g | u] = h W as its second GEMM
  static const char* const names[6] = {"m5_gemm_dh_epilogue", "m6_bwd_reduce", "m7_dy",
                                       "m8_gemm_dW", "m9_gemm_dX", "m10_gemm_dW1"};
  return hip_status(launch_norm_bwd(M, K, d, 2 * F, X, W1, gamma, W, y, r, dgu, dy_in, dX, dW1, dR,
                                    dW, dgamma, ws, wsb + dgu_bytes, names, s));
}

// ------------------------------------------- LM-head GEMM with cross-entropy

namespace {
struct CeWs {
  size_t pmax, psum, lab, total;
  int T;
};
CeWs ce_ws(int64_t M, int64_t V) {
  CeWs w;
  w.T = (int)cdiv(V, coda::kTileN);
  w.pmax = 0;
  w.psum = round_up((size_t)M * w.T * 4);
  w.lab = w.psum + round_up((size_t)M * w.T * 4);
  w.total = w.lab + round_up((size_t)M * 4);
  return w;
}
}  // namespace

size_t coda_ce_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t V) {
  (void)d;
  if (dtype != CODA_BF16 || M < 1 || V < 1) return 0;
  return ce_ws(M, V).total;
}

coda_status coda_ce_fwd(coda_dtype dtype, int64_t M, int64_t d, int64_t V, const void* h,
                        const void* Wv, const int32_t* labels, void* logits, float* lse,
                        float* loss, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!h || !Wv || !labels || !logits || !lse || !loss) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, d) || !dim_ok(dtype, V)) return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, d) || !bytes_ok(dtype, d, V) || !bytes_ok(dtype, M, V))
    return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {h, Wv, (const void*)labels, (const void*)logits, (const void*)lse,
                        (const void*)loss})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const CeWs ws = ce_ws(M, V);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(h, M * d * e), rng(Wv, d * V * e), rng(labels, M * 4)};
  const Range out[] = {rng(logits, M * V * e), rng(lse, M * 4), rng(loss, M * 4),
                       rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  float* pmax = (float*)(wsb + ws.pmax);
  float* psum = (float*)(wsb + ws.psum);
  float* lab = (float*)(wsb + ws.lab);
  hipError_t err;
  // C1: logits = h Wv; epilogue stores them and each tile's (max, sum-exp) per row
  GemmArgs c1 = gemm(M, V, d, h, d, M * d, Wv, V, d * V, logits, V);
  c1.part_row = pmax;
  c1.part_col = psum;
  c1.ld_part_row = ws.T;
  c1.labels = labels;
  c1.lab_out = lab;
  const double Md = 2.0 * M * d, dV = 2.0 * d * V, MV = 2.0 * M * V;
  if ((err = traced("c1_gemm_logits_lse_partials", gemm_flops(M, V, d),
                    Md + dV + MV + 8.0 * M * ws.T + 8.0 * M, s, [&] {
                      return coda::launch_gemm_bf16(c1, true, false, coda::EPI_CE_STATS, s);
                    })) != hipSuccess)
    return hip_status(err);
  // C2: lse and loss from the partials
  return hip_status(traced("c2_ce_combine", 0.0, 8.0 * M * ws.T + 12.0 * M, s, [&] {
    return coda::launch_ce_combine(pmax, psum, ws.T, ws.T, lab, labels, V, M, lse, loss, s);
  }));
}

size_t coda_ce_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t V) {
  (void)d;
  if (dtype != CODA_BF16 || M < 1 || V < 1) return 0;
  return round_up((size_t)M * V * 2);
}

coda_status coda_ce_bwd(coda_dtype dtype, int64_t M, int64_t d, int64_t V, const void* h,
                        const void* Wv, const int32_t* labels, const void* logits,
                        const float* lse, const float* dloss, void* dh, void* dWv,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!h || !Wv || !labels || !logits || !lse || !dloss || !dh || !dWv) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, d) || !dim_ok(dtype, V)) return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, d) || !bytes_ok(dtype, d, V) || !bytes_ok(dtype, M, V))
    return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {h, Wv, (const void*)labels, logits, (const void*)lse,
                        (const void*)dloss, (const void*)dh, (const void*)dWv})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const size_t need = coda_ce_bwd_workspace_bytes(dtype, M, d, V);
  if (!workspace || workspace_bytes < need) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(h, M * d * e), rng(Wv, d * V * e), rng(labels, M * 4),
                      rng(logits, M * V * e), rng(lse, M * 4), rng(dloss, M * 4)};
  const Range out[] = {rng(dh, M * d * e), rng(dWv, d * V * e), rng(workspace, need)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  void* dlog = workspace;
  hipError_t err;
  const double Md = 2.0 * M * d, dV = 2.0 * d * V, MV = 2.0 * M * V;
  // C3: dlogits = dloss (softmax - onehot) from the saved logits and lse
  if ((err = traced("c3_ce_dlogits", 0.0, 2.0 * MV + 12.0 * M, s, [&] {
         return coda::launch_ce_dlogits(logits, labels, lse, dloss, dlog, M, V, s);
       })) != hipSuccess)
    return hip_status(err);
  // C4: dh = dlogits Wv^T
  GemmArgs c4 = gemm(M, d, V, dlog, V, M * V, Wv, V, d * V, dh, d);
  if ((err = traced("c4_gemm_dh", gemm_flops(M, d, V), MV + dV + Md, s, [&] {
         return coda::launch_gemm_bf16(c4, true, true, coda::EPI_STORE, s);
       })) != hipSuccess)
    return hip_status(err);
  // C5: dWv = h^T dlogits
  GemmArgs c5 = gemm(d, V, M, h, d, M * d, dlog, V, M * V, dWv, V);
  return hip_status(traced("c5_gemm_dWv", gemm_flops(d, V, M), Md + MV + dV, s, [&] {
    return coda::launch_gemm_bf16(c5, false, false, coda::EPI_STORE, s);
  }));
}

// --------------------------------------- QKV projection with rotary positions

namespace {
bool rope_args_ok(int64_t N, int64_t N_rot, int64_t D, int64_t S, float base) {
  return D >= 8 && D % 8 == 0 && D <= 4096 && N_rot >= 0 && N_rot <= N && N_rot % D == 0 && S >= 1 &&
         S <= (int64_t)1 << 24 && std::isfinite(base) && base > 0.0f;
}
size_t rope_table_bytes(int64_t D, int64_t S) { return round_up((size_t)S * (size_t)D * 4); }
}  // namespace

size_t coda_rope_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t N,
                                     int64_t N_rot, int64_t D, int64_t S) {
  (void)M;
  (void)K;
  (void)N;
  (void)N_rot;
  if (dtype != CODA_BF16 || D < 1 || S < 1) return 0;
  return rope_table_bytes(D, S);
}

coda_status coda_rope_fwd(coda_dtype dtype, int64_t M, int64_t K, int64_t N, int64_t N_rot,
                          int64_t D, int64_t S, float base, const void* X, const void* W, void* Y,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W || !Y) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, K) || !dim_ok(dtype, N)) return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, K) || !bytes_ok(dtype, K, N) || !bytes_ok(dtype, M, N))
    return CODA_ERR_SHAPE;
  if (!rope_args_ok(N, N_rot, D, S, base)) return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W, (const void*)Y})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const size_t tb = rope_table_bytes(D, S);
  if (!workspace || workspace_bytes < tb) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W, K * N * e)};
  const Range out[] = {rng(Y, M * N * e), rng(workspace, tb)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  float* tab = (float*)workspace;
  hipError_t err;
  if ((err = traced("q0_rope_table", 0.0, (double)S * D * 4.0, s, [&] {
         return coda::launch_rope_table(tab, (int)S, (int)D, (double)base, s);
       })) != hipSuccess)
    return hip_status(err);
  // Q1: Y = rope(X W), the rotation in the epilogue
  GemmArgs q1 = gemm(M, N, K, X, K, M * K, W, N, K * N, Y, N);
  q1.rope_tab = tab;
  q1.rope_rot = (int)N_rot;
  q1.rope_head = (int)D;
  q1.rope_seq = (int)S;
  const double mk = 2.0 * M * K, kn = 2.0 * K * N, mn = 2.0 * M * N;
  return hip_status(traced("q1_gemm_qkv_rope", gemm_flops(M, N, K), mk + kn + mn + (double)S * D * 4.0, s,
                           [&] { return coda::launch_gemm_bf16(q1, true, false, coda::EPI_ROPE, s); }));
}

size_t coda_rope_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t N,
                                     int64_t N_rot, int64_t D, int64_t S) {
  (void)K;
  (void)N_rot;
  if (dtype != CODA_BF16 || M < 1 || N < 1 || D < 1 || S < 1) return 0;
  return rope_table_bytes(D, S) + round_up((size_t)M * N * 2);
}

coda_status coda_rope_bwd(coda_dtype dtype, int64_t M, int64_t K, int64_t N, int64_t N_rot,
                          int64_t D, int64_t S, float base, const void* X, const void* W,
                          const void* dY, void* dX, void* dW, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return CODA_ERR_DTYPE;
  if (!X || !W || !dY || !dX || !dW) return CODA_ERR_NULL;
  if (!rows_ok(dtype, M) || !dim_ok(dtype, K) || !dim_ok(dtype, N)) return CODA_ERR_SHAPE;
  if (!bytes_ok(dtype, M, K) || !bytes_ok(dtype, K, N) || !bytes_ok(dtype, M, N))
    return CODA_ERR_SHAPE;
  if (!rope_args_ok(N, N_rot, D, S, base)) return CODA_ERR_SHAPE;
  if (dtype != CODA_BF16) return CODA_ERR_UNSUPPORTED;
  for (const void* p : {X, W, dY, (const void*)dX, (const void*)dW})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const size_t tb = rope_table_bytes(D, S);
  const size_t need = tb + round_up((size_t)M * N * 2);
  if (!workspace || workspace_bytes < need) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W, K * N * e), rng(dY, M * N * e)};
  const Range out[] = {rng(dX, M * K * e), rng(dW, K * N * e), rng(workspace, need)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  float* tab = (float*)workspace;
  void* dP = (char*)workspace + tb;
  hipError_t err;
  const double mk = 2.0 * M * K, kn = 2.0 * K * N, mn = 2.0 * M * N;
  if ((err = traced("q2_rope_table", 0.0, (double)S * D * 4.0, s, [&] {
         return coda::launch_rope_table(tab, (int)S, (int)D, (double)base, s);
       })) != hipSuccess)
    return hip_status(err);
  // Q3: dP = the transposed rotation of dY
  if ((err = traced("q3_rope_inverse", 0.0, 2.0 * mn + (double)S * D * 4.0, s, [&] {
         return coda::launch_rope_inverse(dY, tab, dP, M, N, (int)N_rot, (int)D, (int)S, s);
       })) != hipSuccess)
    return hip_status(err);
  // Q4: dX = dP W^T
  GemmArgs q4 = gemm(M, K, N, dP, N, M * N, W, N, K * N, dX, K);
  if ((err = traced("q4_gemm_dX", gemm_flops(M, K, N), mn + kn + mk, s, [&] {
         return coda::launch_gemm_bf16(q4, true, true, coda::EPI_STORE, s);
       })) != hipSuccess)
    return hip_status(err);
  // Q5: dW = X^T dP
  GemmArgs q5 = gemm(K, N, M, X, K, M * K, dP, N, M * N, dW, N);
  return hip_status(traced("q5_gemm_dW", gemm_flops(K, N, M), mk + mn + kn, s, [&] {
    return coda::launch_gemm_bf16(q5, false, false, coda::EPI_STORE, s);
  }));
}

coda_status coda_mx8_quantize(int64_t rows, int64_t cols, const void* src, int64_t ld_src,
                              void* codes, void* scales, void* stream) {
  if (!src || !codes || !scales) return CODA_ERR_NULL;
  if (rows < 1 || !mx_dim_ok(cols, 128) || ld_src < cols || ld_src % 8 != 0 || ld_src > kMaxRowLen ||
      rows > kMaxRows)
    return CODA_ERR_SHAPE;
  if (!fits(rows, ld_src, 2) || !fits(rows, cols, 1) || !scales_fit(rows, cols)) return CODA_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(codes)) return CODA_ERR_ALIGN;
  const Range in[] = {rng(src, ((rows - 1) * ld_src + cols) * 2)};
  const Range out[] = {rng(codes, rows * cols), rng(scales, rows * (cols / 32))};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  return hip_status(traced("x0_mx8_quantize", 0.0, rows * cols * (3.0 + 1.0 / 32.0), s, [&] {
    return coda::launch_mx8_quantize(src, ld_src, rows, cols, (uint8_t*)codes, (uint8_t*)scales, s);
  }));
}

size_t coda_fwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t N) {
  (void)K;
  (void)N;
  if (M < 1 || d < 32 || d % 32 != 0) return 0;
  return mx8_ws(M, d).total;
}

coda_status coda_fwd_mx8(int64_t M, int64_t K, int64_t d, int64_t N, float eps, const void* Xq,
                         const void* Xs, const void* W1tq, const void* W1ts, const void* R,
                         const void* gamma, const void* W2tq, const void* W2ts, void* y, float* r,
                         void* z, void* workspace, size_t workspace_bytes, void* stream) {
  if (!Xq || !Xs || !W1tq || !W1ts || !R || !gamma || !W2tq || !W2ts || !y || !r || !z)
    return CODA_ERR_NULL;
  if (!mx_rows_ok(M, 8) || !mx_dim_ok(N, 8) || !mx_dim_ok(K, 128) || !mx_dim_ok(d, 128))
    return CODA_ERR_SHAPE;
  if (!fits(M, K, 1) || !fits(d, K, 1) || !fits(N, d, 1) || !fits(M, d, 2) || !fits(M, N, 2) ||
      !scales_fit(M, K) || !scales_fit(d, K) || !scales_fit(N, d) || !scales_fit(M, d))
    return CODA_ERR_SHAPE;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return CODA_ERR_EPS;
  for (const void* p : {Xq, Xs, W1tq, W1ts, R, gamma, W2tq, W2ts, (const void*)y, (const void*)r,
                        (const void*)z})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const Mx8Ws ws = mx8_ws(M, d);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const Range in[] = {rng(Xq, M * K), rng(Xs, M * (K / 32)), rng(W1tq, d * K), rng(W1ts, d * (K / 32)),
                      rng(R, M * d * 2), rng(gamma, d * 2), rng(W2tq, N * d), rng(W2ts, N * (d / 32))};
  const Range out[] = {rng(y, M * d * 2), rng(r, M * 4), rng(z, M * N * 2), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  float* P = (float*)(wsb + ws.P);
  uint8_t* q = (uint8_t*)(wsb + ws.q);
  uint8_t* qs = (uint8_t*)(wsb + ws.qs);
  hipError_t err;
  // K1: y = deq(X) deq(W1t)^T + R; epilogue: y (bf16), partial sums, y gamma as MXFP8
  GemmArgs g1 = gemm_mx8(M, d, K, Xq, Xs, W1tq, W1ts, y, d);
  g1.E = R;
  g1.lde = d;
  g1.part_row = P;
  g1.ld_part_row = ws.Tn;
  g1.vcol = gamma;
  g1.q_out = q;
  g1.qs_out = qs;
  g1.ldq = d;
  const double k1_bytes = (M + d) * K * (1.0 + 1.0 / 32.0) + 4.0 * M * d + M * d * (1.0 + 1.0 / 32.0) +
                          M * ws.Tn * 4.0 + 2.0 * d;
  if ((err = traced("k1_gemm_mx8_resid_sumsq", gemm_flops(M, d, K), k1_bytes, s, [&] {
         return coda::launch_gemm_mx8(g1, coda::EPI_RESID_SUMSQ, s);
       })) != hipSuccess)
    return hip_status(err);
  // K2: z = diag(r) (deq(q) deq(W2t)^T); r from the partial sums in the epilogue
  GemmArgs g2 = gemm_mx8(M, N, d, q, qs, W2tq, W2ts, z, N);
  g2.part_row = P;
  g2.ld_part_row = ws.Tn;
  g2.nparts = ws.Tn;
  g2.inv_d = 1.0f / (float)d;
  g2.eps = eps;
  g2.r_out = r;
  const double k2_bytes = (M + N) * d * (1.0 + 1.0 / 32.0) + 2.0 * M * N + M * ws.Tn * 4.0 + 4.0 * M;
  return hip_status(traced("k2_gemm_mx8_rsqrt_rowscale", gemm_flops(M, N, d), k2_bytes, s, [&] {
    return coda::launch_gemm_mx8(g2, coda::EPI_RSQRT_SCALE, s);
  }));
}

// ------------------------------------------------------ MXFP8 backward

}  // extern "C"

namespace {
// Workspace of coda_bwd_mx8: every GEMM operand in MXFP8 (codes, then
// step-blocked scales), plus n (bf16) and the partial sums of the bf16
// backward.
struct BwdMx8Ws {
  size_t dzq, dzs, w2q, w2s, S, G, c, nTq, nTs, dzTq, dzTs, dyq, dys, w1q, w1s, XTq, XTs, dyTq, dyTs, total;
  int Tn, Tm;
};
BwdMx8Ws bwd_mx8_ws(int64_t M, int64_t K, int64_t d, int64_t N) {
  BwdMx8Ws w;
  w.Tn = (int)cdiv(d, coda::kTileN);
  w.Tm = (int)cdiv(M, coda::kTileM);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes); return at; };
  w.dzq = take((size_t)M * N);       w.dzs = take((size_t)M * (N / 32));
  w.w2q = take((size_t)d * N);       w.w2s = take((size_t)d * (N / 32));
  w.S = take((size_t)M * w.Tn * 4);  w.G = take((size_t)w.Tm * d * 4);  w.c = take((size_t)M * 4);
  w.nTq = take((size_t)d * M);       w.nTs = take((size_t)d * (M / 32));
  w.dzTq = take((size_t)N * M);      w.dzTs = take((size_t)N * (M / 32));
  w.dyq = take((size_t)M * d);       w.dys = take((size_t)M * (d / 32));
  w.w1q = take((size_t)K * d);       w.w1s = take((size_t)K * (d / 32));
  w.XTq = take((size_t)K * M);       w.XTs = take((size_t)K * (M / 32));
  w.dyTq = take((size_t)d * M);      w.dyTs = take((size_t)d * (M / 32));
  w.total = o;
  return w;
}

// The MXFP8 backward of the block (coda_bwd_mx8; the MLP sub-layer's second
// half with W2 = W, dz = dgu and dy_in): every argument already checked.  dz
// NULL: dz's MXFP8 operands (along N and along M) are already in the
// workspace.
coda_status norm_bwd_mx8(int64_t M, int64_t K, int64_t d, int64_t N, const void* X, const void* W1,
                         const void* gamma, const void* W2, const void* y, const float* r, const void* dz,
                         const void* dy_in, void* dX, void* dW1, void* dR, void* dW2, float* dgamma,
                         void* workspace, const BwdMx8Ws& ws, hipStream_t s) {
  const size_t e = 2;
  char* wb = (char*)workspace;
  auto u8 = [&](size_t off) { return (uint8_t*)(wb + off); };
  float* S = (float*)(wb + ws.S);
  float* G = (float*)(wb + ws.G);
  float* c = (float*)(wb + ws.c);
  hipError_t err;
  const double md = (double)M * d, mn = (double)M * N, dn2 = (double)d * N, mk = (double)M * K, kd = (double)K * d;
  const double q8 = 1.0 + 1.0 / 32.0;   // MXFP8 bytes per element (code + a scale per 32)
  auto quant = [&](const char* name, const void* src, int64_t rows, int64_t cols, uint8_t* q, uint8_t* qs) {
    return traced(name, 0.0, rows * cols * (2.0 + q8), s, [&] {
      return coda::launch_mx8_quantize(src, cols, rows, cols, q, qs, s);
    });
  };
  auto fused = [&](const char* name, double bytes, int mode, const coda::MxQuantArgs& q) {
    return traced(name, 0.0, bytes, s, [&] { return coda::launch_mx8_quantize_fused(q, mode, s); });
  };
  auto qargs = [&](const void* src, int64_t rows, int64_t cols) {
    coda::MxQuantArgs q{};
    q.src = src;
    q.ld = cols;
    q.rows = rows;
    q.cols = cols;
    return q;
  };
  // dz along N (the dh GEMM's contraction index) and along M, stored
  // transposed (the dW2 GEMM's), in one pass; W2 along N
  coda::MxQuantArgs qdz = qargs(dz, M, N);
  qdz.qr = u8(ws.dzq);
  qdz.sr = u8(ws.dzs);
  qdz.qt = u8(ws.dzTq);
  qdz.st = u8(ws.dzTs);
  // (dz NULL: its codes are already in the workspace, written by the GEMM
  // that produced it)
  if (dz && (err = fused("x1_mx8_quantize_dz_both", mn * (2.0 + 2.0 * q8), 0, qdz)) != hipSuccess)
    return hip_status(err);
  if ((err = quant("x2_mx8_quantize_W2", W2, d, N, u8(ws.w2q), u8(ws.w2s))) != hipSuccess) return hip_status(err);
  // B1: dh = dz W2^T on MXFP8; epilogue dn (into dR), S, G as in the bf16
  // backward (n is made from y and r where it is quantised)
  GemmArgs b1 = gemm_mx8(M, d, N, u8(ws.dzq), u8(ws.dzs), u8(ws.w2q), u8(ws.w2s), dR, d);
  b1.E = y;
  b1.lde = d;
  b1.vrow = r;
  b1.vcol = gamma;
  b1.part_row = S;
  b1.ld_part_row = ws.Tn;
  b1.part_col = G;
  b1.ld_part_col = d;
  if ((err = traced("b1_gemm_mx8_dh_epilogue", gemm_flops(M, d, N),
                    (mn + dn2) * q8 + 2.0 * md * e + M * ws.Tn * 4.0 + ws.Tm * d * 4.0 + 4.0 * M, s,
                    [&] { return coda::launch_gemm_mx8(b1, coda::EPI_DN, s); })) != hipSuccess)
    return hip_status(err);
  // R2 as in the bf16 backward
  if ((err = traced("r2_bwd_reduce", 0.0, M * ws.Tn * 4.0 + ws.Tm * d * 4.0 + 8.0 * M + 4.0 * d, s, [&] {
         return coda::launch_bwd_reduce(S, ws.Tn, ws.Tn, r, M, d, G, ws.Tm, c, dgamma, s);
       })) != hipSuccess)
    return hip_status(err);
  // E2 with the quantisations of dy: dy = r dn - c y written over dn (dR),
  // then along d (the dX GEMM's contraction index) and along M, transposed
  // (the dW1 GEMM's)
  coda::MxQuantArgs qdy = qargs(dR, M, d);
  qdy.r = r;
  qdy.c = c;
  qdy.y = y;
  qdy.dy_in = dy_in;
  qdy.out = dR;
  qdy.qr = u8(ws.dyq);
  qdy.sr = u8(ws.dys);
  qdy.qt = u8(ws.dyTq);
  qdy.st = u8(ws.dyTs);
  if ((err = fused("e2_dy_mx8_quantize_both", md * (3.0 * e + 2.0 * q8) + 8.0 * M, 1, qdy)) != hipSuccess)
    return hip_status(err);
  // B2: dW2 = diag(gamma) n^T dz, contraction over M: n = r y (bf16) along M,
  // transposed
  coda::MxQuantArgs qn = qargs(y, M, d);
  qn.r = r;
  qn.qt = u8(ws.nTq);
  qn.st = u8(ws.nTs);
  if ((err = fused("x3_mx8_quantize_nT", md * (e + q8) + 4.0 * M, 2, qn)) != hipSuccess) return hip_status(err);
  GemmArgs b2 = gemm_mx8(d, N, M, u8(ws.nTq), u8(ws.nTs), u8(ws.dzTq), u8(ws.dzTs), dW2, N);
  b2.vcol = gamma;
  if ((err = traced("b2_gemm_mx8_dW2", gemm_flops(d, N, M), (md + mn) * q8 + dn2 * e + 2.0 * d, s,
                    [&] { return coda::launch_gemm_mx8(b2, coda::EPI_ROWSCALE, s); })) != hipSuccess)
    return hip_status(err);
  // B3: dX = dy W1^T, contraction over d: W1 along d
  if ((err = quant("x6_mx8_quantize_W1", W1, K, d, u8(ws.w1q), u8(ws.w1s))) != hipSuccess) return hip_status(err);
  GemmArgs b3 = gemm_mx8(M, K, d, u8(ws.dyq), u8(ws.dys), u8(ws.w1q), u8(ws.w1s), dX, K);
  if ((err = traced("b3_gemm_mx8_dX", gemm_flops(M, K, d), (md + kd) * q8 + mk * e, s,
                    [&] { return coda::launch_gemm_mx8(b3, coda::EPI_STORE, s); })) != hipSuccess)
    return hip_status(err);
  // B4: dW1 = X^T dy, contraction over M: X along M, transposed
  if ((err = traced("x7_mx8_quantize_XT", 0.0, mk * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(X, K, M, K, u8(ws.XTq), u8(ws.XTs), s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs b4 = gemm_mx8(K, d, M, u8(ws.XTq), u8(ws.XTs), u8(ws.dyTq), u8(ws.dyTs), dW1, d);
  return hip_status(traced("b4_gemm_mx8_dW1", gemm_flops(K, d, M), (mk + md) * q8 + kd * e, s,
                           [&] { return coda::launch_gemm_mx8(b4, coda::EPI_STORE, s); }));
}
}  // namespace

extern "C" {

size_t coda_bwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t N) {
  if (M < 128 || K < 8 || d < 128 || N < 128 || M % 128 || d % 128 || N % 128) return 0;
  return bwd_mx8_ws(M, K, d, N).total;
}

coda_status coda_bwd_mx8(int64_t M, int64_t K, int64_t d, int64_t N, const void* X, const void* W1,
                         const void* gamma, const void* W2, const void* y, const float* r,
                         const void* dz, void* dX, void* dW1, void* dR, void* dW2, float* dgamma,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !W1 || !gamma || !W2 || !y || !r || !dz || !dX || !dW1 || !dR || !dW2 || !dgamma)
    return CODA_ERR_NULL;
  // the contraction dimensions of the four GEMMs (N, M, d) are whole K steps
  if (!mx_rows_ok(M, 128) || !mx_dim_ok(K, 8) || !mx_dim_ok(d, 128) || !mx_dim_ok(N, 128))
    return CODA_ERR_SHAPE;
  if (!fits(M, K, 2) || !fits(K, d, 2) || !fits(M, d, 2) || !fits(d, N, 2) || !fits(M, N, 2) ||
      !scales_fit(M, N) || !scales_fit(d, N) || !scales_fit(N, M) || !scales_fit(d, M) ||
      !scales_fit(M, d) || !scales_fit(K, d) || !scales_fit(K, M))
    return CODA_ERR_SHAPE;
  for (const void* p : {X, W1, gamma, W2, y, (const void*)r, dz, (const void*)dX, (const void*)dW1,
                        (const void*)dR, (const void*)dW2, (const void*)dgamma})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const BwdMx8Ws ws = bwd_mx8_ws(M, K, d, N);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(gamma, d * e), rng(W2, d * N * e),
                      rng(y, M * d * e), rng(r, M * 4), rng(dz, M * N * e)};
  const Range out[] = {rng(dX, M * K * e), rng(dW1, K * d * e), rng(dR, M * d * e),
                       rng(dW2, d * N * e), rng(dgamma, d * 4), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  return norm_bwd_mx8(M, K, d, N, X, W1, gamma, W2, y, r, dz, nullptr, dX, dW1, dR, dW2, dgamma, workspace, ws,
                      (hipStream_t)stream);
}

}  // extern "C"

namespace {
// Workspaces of the MXFP8 SwiGLU block: every GEMM operand in MXFP8 (codes
// and step-blocked scales; dgu exists only as such).
struct SwigluMx8Ws {
  size_t xq, xs, wq, ws, wdq, wds, aq, as, total;          // forward
  size_t dzq, dzs, dzTq, dzTs, wdrq, wdrs, aTq, aTs, dguq, dgus, dguTq, dguTs, wrq, wrs, XTq, XTs;
};
SwigluMx8Ws swiglu_mx8_ws(int64_t M, int64_t d, int64_t F, bool bwd) {
  SwigluMx8Ws w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes); return at; };
  auto mx = [&](size_t rows, size_t k, size_t& q, size_t& sc) { q = take(rows * k); sc = take(rows * (k / 32)); };
  if (!bwd) {
    mx(M, d, w.xq, w.xs);            // X along d
    mx(2 * F, d, w.wq, w.ws);        // W along d, transposed, gate/up order
    mx(d, F, w.wdq, w.wds);          // Wd along F, transposed
    mx(M, F, w.aq, w.as);            // a along F (from the gate/up GEMM's epilogue)
  } else {
    mx(M, d, w.dzq, w.dzs);          // dz along d
    mx(d, M, w.dzTq, w.dzTs);        // dz along M, transposed
    mx(F, d, w.wdrq, w.wdrs);        // Wd along d
    mx(F, M, w.aTq, w.aTs);          // a along M, transposed
    mx(M, 2 * F, w.dguq, w.dgus);    // dgu along 2F
    mx(2 * F, M, w.dguTq, w.dguTs);  // dgu along M, transposed
    mx(d, 2 * F, w.wrq, w.wrs);      // W along 2F
    mx(d, M, w.XTq, w.XTs);          // X along M, transposed
  }
  w.total = o;
  return w;
}
bool swiglu_mx8_shape_ok(int64_t M, int64_t d, int64_t F) {
  return mx_rows_ok(M, 128) && mx_dim_ok(d, 128) && mx_dim_ok(F, 128) && mx_dim_ok(2 * F, 128) &&
         fits(M, 2 * F, 2) && fits(d, 2 * F, 2) && scales_fit(M, 2 * F) && scales_fit(2 * F, M) &&
         scales_fit(d, 2 * F) && scales_fit(2 * F, d) && scales_fit(M, d) && scales_fit(d, M) &&
         scales_fit(F, M) && scales_fit(M, F) && scales_fit(F, d) && scales_fit(d, F);
}
}  // namespace

extern "C" {

size_t coda_swiglu_fwd_mx8_workspace_bytes(int64_t M, int64_t d, int64_t F) {
  if (!swiglu_mx8_shape_ok(M, d, F)) return 0;
  return swiglu_mx8_ws(M, d, F, false).total;
}

size_t coda_swiglu_bwd_mx8_workspace_bytes(int64_t M, int64_t d, int64_t F) {
  if (!swiglu_mx8_shape_ok(M, d, F)) return 0;
  return swiglu_mx8_ws(M, d, F, true).total;
}

coda_status coda_swiglu_fwd_mx8(int64_t M, int64_t d, int64_t F, const void* X, const void* W,
                                const void* Wd, void* gu, void* a, void* z, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!X || !W || !Wd || !gu || !a || !z) return CODA_ERR_NULL;
  if (!swiglu_mx8_shape_ok(M, d, F)) return CODA_ERR_SHAPE;
  for (const void* p : {X, W, Wd, (const void*)gu, (const void*)a, (const void*)z})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const SwigluMx8Ws ws = swiglu_mx8_ws(M, d, F, false);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * d * e), rng(W, d * 2 * F * e), rng(Wd, F * d * e)};
  const Range out[] = {rng(gu, M * 2 * F * e), rng(a, M * F * e), rng(z, M * d * e), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wb = (char*)workspace;
  auto u8 = [&](size_t off) { return (uint8_t*)(wb + off); };
  hipError_t err;
  const double q8 = 1.0 + 1.0 / 32.0, Md = (double)M * d, dF = (double)d * F, MF = (double)M * F;
  // operands: X along d; W along d, transposed into gate/up order; Wd along F, transposed
  if ((err = traced("x1_mx8_quantize_X", 0.0, Md * (e + q8), s, [&] {
         return coda::launch_mx8_quantize(X, d, M, d, u8(ws.xq), u8(ws.xs), s);
       })) != hipSuccess)
    return hip_status(err);
  coda::MxQuantArgs qw{};
  qw.src = W;
  qw.ld = 2 * F;
  qw.rows = d;
  qw.cols = 2 * F;
  qw.qt = u8(ws.wq);
  qw.st = u8(ws.ws);
  qw.gated_F = F;
  if ((err = traced("x2_mx8_quantize_W_gateup", 0.0, 2.0 * dF * (e + q8), s,
                    [&] { return coda::launch_mx8_quantize_fused(qw, 0, s); })) != hipSuccess)
    return hip_status(err);
  if ((err = traced("x3_mx8_quantize_WdT", 0.0, dF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(Wd, d, F, d, u8(ws.wdq), u8(ws.wds), s);
       })) != hipSuccess)
    return hip_status(err);
  // S1: [g | u] = X W on MXFP8; epilogue gu, a = silu(g) u (bf16) and a to MXFP8 along F
  GemmArgs s1 = gemm_mx8(M, F, d, u8(ws.xq), u8(ws.xs), u8(ws.wq), u8(ws.ws), gu, 2 * F);
  s1.B_total = (uint64_t)(2 * F * d);
  s1.B_bytes = (uint32_t)std::min<uint64_t>(s1.B_total, 0x7FFFFFF0ull);
  s1.sB_bytes = (uint32_t)(2 * F * (d / 32));
  s1.C2 = a;
  s1.ldc2 = F;
  s1.F = (int)F;
  s1.q_out = u8(ws.aq);
  s1.qs_out = u8(ws.as);
  s1.ldq = F;
  if ((err = traced("s1_gemm_mx8_gateup_swiglu", gemm_flops(M, 2 * F, d),
                    (Md + 2.0 * dF) * q8 + 3.0 * MF * e + MF * q8, s,
                    [&] { return coda::launch_gemm_mx8(s1, coda::EPI_SWIGLU, s); })) != hipSuccess)
    return hip_status(err);
  // S2: z = a Wd on MXFP8
  GemmArgs s2 = gemm_mx8(M, d, F, u8(ws.aq), u8(ws.as), u8(ws.wdq), u8(ws.wds), z, d);
  return hip_status(traced("s2_gemm_mx8_down", gemm_flops(M, d, F), (MF + dF) * q8 + Md * e, s,
                           [&] { return coda::launch_gemm_mx8(s2, coda::EPI_STORE, s); }));
}

coda_status coda_swiglu_bwd_mx8(int64_t M, int64_t d, int64_t F, const void* X, const void* W,
                                const void* Wd, const void* gu, const void* a, const void* dz, void* dX,
                                void* dW, void* dWd, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!X || !W || !Wd || !gu || !a || !dz || !dX || !dW || !dWd) return CODA_ERR_NULL;
  if (!swiglu_mx8_shape_ok(M, d, F)) return CODA_ERR_SHAPE;
  for (const void* p : {X, W, Wd, gu, a, dz, (const void*)dX, (const void*)dW, (const void*)dWd})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const SwigluMx8Ws ws = swiglu_mx8_ws(M, d, F, true);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * d * e), rng(W, d * 2 * F * e), rng(Wd, F * d * e),
                      rng(gu, M * 2 * F * e), rng(a, M * F * e), rng(dz, M * d * e)};
  const Range out[] = {rng(dX, M * d * e), rng(dW, d * 2 * F * e), rng(dWd, F * d * e),
                       rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wb = (char*)workspace;
  auto u8 = [&](size_t off) { return (uint8_t*)(wb + off); };
  hipError_t err;
  const double q8 = 1.0 + 1.0 / 32.0, Md = (double)M * d, dF = (double)d * F, MF = (double)M * F;
  auto both = [&](const char* name, const void* src, int64_t rows, int64_t cols, size_t qr, size_t sr, size_t qt,
                  size_t st) {
    coda::MxQuantArgs q{};
    q.src = src;
    q.ld = cols;
    q.rows = rows;
    q.cols = cols;
    q.qr = u8(qr);
    q.sr = u8(sr);
    q.qt = u8(qt);
    q.st = u8(st);
    return traced(name, 0.0, (double)rows * cols * (e + 2.0 * q8), s,
                  [&] { return coda::launch_mx8_quantize_fused(q, 0, s); });
  };
  // S3: da = dz Wd^T (contraction over d); epilogue dgu from the saved gu
  if ((err = both("x1_mx8_quantize_dz_both", dz, M, d, ws.dzq, ws.dzs, ws.dzTq, ws.dzTs)) != hipSuccess)
    return hip_status(err);
  if ((err = traced("x2_mx8_quantize_Wd", 0.0, dF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize(Wd, d, F, d, u8(ws.wdrq), u8(ws.wdrs), s);
       })) != hipSuccess)
    return hip_status(err);
  // (dgu is not stored: the epilogue quantises it, as bf16, along 2F and
  // along M for the dX and dW GEMMs)
  GemmArgs s3 = gemm_mx8(M, F, d, u8(ws.dzq), u8(ws.dzs), u8(ws.wdrq), u8(ws.wdrs), nullptr, 2 * F);
  s3.E = gu;
  s3.lde = 2 * F;
  s3.F = (int)F;
  s3.q_out = u8(ws.dguq);
  s3.qs_out = u8(ws.dgus);
  s3.ldq = 2 * F;
  s3.qt_out = u8(ws.dguTq);
  s3.qts_out = u8(ws.dguTs);
  s3.ldqt = M;
  if ((err = traced("s3_gemm_mx8_da_swiglu_bwd", gemm_flops(M, F, d), (Md + dF) * q8 + 2.0 * MF * e + 4.0 * MF * q8,
                    s, [&] { return coda::launch_gemm_mx8(s3, coda::EPI_SWIGLU_BWD, s); })) != hipSuccess)
    return hip_status(err);
  // S4: dWd = a^T dz (contraction over M): a along M, transposed
  if ((err = traced("x3_mx8_quantize_aT", 0.0, MF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(a, F, M, F, u8(ws.aTq), u8(ws.aTs), s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs s4 = gemm_mx8(F, d, M, u8(ws.aTq), u8(ws.aTs), u8(ws.dzTq), u8(ws.dzTs), dWd, d);
  if ((err = traced("s4_gemm_mx8_dWd", gemm_flops(F, d, M), (MF + Md) * q8 + dF * e, s,
                    [&] { return coda::launch_gemm_mx8(s4, coda::EPI_STORE, s); })) != hipSuccess)
    return hip_status(err);
  // S5: dX = dgu W^T (contraction over 2F); S6: dW = X^T dgu (contraction over M)
  if ((err = traced("x5_mx8_quantize_W", 0.0, 2.0 * dF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize(W, 2 * F, d, 2 * F, u8(ws.wrq), u8(ws.wrs), s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs s5 = gemm_mx8(M, d, 2 * F, u8(ws.dguq), u8(ws.dgus), u8(ws.wrq), u8(ws.wrs), dX, d);
  if ((err = traced("s5_gemm_mx8_dX", gemm_flops(M, d, 2 * F), (2.0 * MF + 2.0 * dF) * q8 + Md * e, s,
                    [&] { return coda::launch_gemm_mx8(s5, coda::EPI_STORE, s); })) != hipSuccess)
    return hip_status(err);
  if ((err = traced("x6_mx8_quantize_XT", 0.0, Md * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(X, d, M, d, u8(ws.XTq), u8(ws.XTs), s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs s6 = gemm_mx8(d, 2 * F, M, u8(ws.XTq), u8(ws.XTs), u8(ws.dguTq), u8(ws.dguTs), dW, 2 * F);
  return hip_status(traced("s6_gemm_mx8_dW", gemm_flops(d, 2 * F, M), (Md + 2.0 * MF) * q8 + 2.0 * dF * e, s,
                           [&] { return coda::launch_gemm_mx8(s6, coda::EPI_STORE, s); }));
}

// --------------------------------------------------- MXFP8 MLP sub-layer

}  // extern "C"

namespace {
struct MlpMx8FwdWs {
  size_t xq, xs, w1q, w1s, P, ygq, ygs, wq, ws, wdq, wds, aq, as, total;
  int Tn;
};
MlpMx8FwdWs mlp_mx8_fwd_ws(int64_t M, int64_t K, int64_t d, int64_t F) {
  MlpMx8FwdWs w{};
  w.Tn = (int)cdiv(d, coda::kTileN);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes); return at; };
  auto mx = [&](size_t rows, size_t k, size_t& q, size_t& sc) { q = take(rows * k); sc = take(rows * (k / 32)); };
  mx(M, K, w.xq, w.xs);          // X along K
  mx(d, K, w.w1q, w.w1s);        // W1 along K, transposed
  w.P = take((size_t)M * w.Tn * 4);
  mx(M, d, w.ygq, w.ygs);        // y gamma along d (the first GEMM's epilogue)
  mx(2 * F, d, w.wq, w.ws);      // W along d, transposed, gate/up order
  mx(d, F, w.wdq, w.wds);        // Wd along F, transposed
  mx(M, F, w.aq, w.as);          // a along F (the gate/up GEMM's epilogue)
  w.total = o;
  return w;
}
// The backward: the SwiGLU part's operands, then the block part's workspace
// (coda_bwd_mx8's with N = 2F; its dz operands receive dgu's codes)
struct MlpMx8BwdWs {
  size_t dzq, dzs, dzTq, dzTs, wdq, wds, aTq, aTs, blk, total;
  BwdMx8Ws b;
};
MlpMx8BwdWs mlp_mx8_bwd_ws(int64_t M, int64_t K, int64_t d, int64_t F) {
  MlpMx8BwdWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes); return at; };
  auto mx = [&](size_t rows, size_t k, size_t& q, size_t& sc) { q = take(rows * k); sc = take(rows * (k / 32)); };
  mx(M, d, w.dzq, w.dzs);
  mx(d, M, w.dzTq, w.dzTs);
  mx(F, d, w.wdq, w.wds);
  mx(F, M, w.aTq, w.aTs);
  w.b = bwd_mx8_ws(M, K, d, 2 * F);
  w.blk = take(w.b.total);
  w.total = o;
  return w;
}
bool mlp_mx8_shape_ok(int64_t M, int64_t K, int64_t d, int64_t F) {
  return mx_rows_ok(M, 128) && mx_dim_ok(K, 128) && swiglu_mx8_shape_ok(M, d, F) && fits(M, K, 2) &&
         fits(K, d, 2) && scales_fit(M, K) && scales_fit(d, K) && scales_fit(K, d) && scales_fit(K, M);
}
}  // namespace

extern "C" {

size_t coda_mlp_fwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t F) {
  if (!mlp_mx8_shape_ok(M, K, d, F)) return 0;
  return mlp_mx8_fwd_ws(M, K, d, F).total;
}

size_t coda_mlp_bwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t F) {
  if (!mlp_mx8_shape_ok(M, K, d, F)) return 0;
  return mlp_mx8_bwd_ws(M, K, d, F).total;
}

coda_status coda_mlp_fwd_mx8(int64_t M, int64_t K, int64_t d, int64_t F, float eps, const void* X,
                             const void* W1, const void* R, const void* gamma, const void* W, const void* Wd,
                             void* y, float* r, void* gu, void* a, void* z, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!X || !W1 || !R || !gamma || !W || !Wd || !y || !r || !gu || !a || !z) return CODA_ERR_NULL;
  if (!mlp_mx8_shape_ok(M, K, d, F)) return CODA_ERR_SHAPE;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return CODA_ERR_EPS;
  for (const void* p : {X, W1, R, gamma, W, Wd, (const void*)y, (const void*)r, (const void*)gu, (const void*)a,
                        (const void*)z})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  const MlpMx8FwdWs ws = mlp_mx8_fwd_ws(M, K, d, F);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(R, M * d * e), rng(gamma, d * e),
                      rng(W, d * 2 * F * e), rng(Wd, F * d * e)};
  const Range out[] = {rng(y, M * d * e), rng(r, M * 4), rng(gu, M * 2 * F * e), rng(a, M * F * e),
                       rng(z, M * d * e), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wb = (char*)workspace;
  auto u8 = [&](size_t off) { return (uint8_t*)(wb + off); };
  float* P = (float*)(wb + ws.P);
  hipError_t err;
  const double q8 = 1.0 + 1.0 / 32.0, MK = (double)M * K, Kd = (double)K * d, Md = (double)M * d,
               dF = (double)d * F, MF = (double)M * F;
  // operands: X along K; W1 along K, transposed
  if ((err = traced("x1_mx8_quantize_X", 0.0, MK * (e + q8), s, [&] {
         return coda::launch_mx8_quantize(X, K, M, K, u8(ws.xq), u8(ws.xs), s);
       })) != hipSuccess)
    return hip_status(err);
  if ((err = traced("x2_mx8_quantize_W1T", 0.0, Kd * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(W1, d, K, d, u8(ws.w1q), u8(ws.w1s), s);
       })) != hipSuccess)
    return hip_status(err);
  // K1: y = X W1 + R on MXFP8; epilogue y, partial sums, y gamma along d
  GemmArgs g1 = gemm_mx8(M, d, K, u8(ws.xq), u8(ws.xs), u8(ws.w1q), u8(ws.w1s), y, d);
  g1.E = R;
  g1.lde = d;
  g1.part_row = P;
  g1.ld_part_row = ws.Tn;
  g1.vcol = gamma;
  g1.q_out = u8(ws.ygq);
  g1.qs_out = u8(ws.ygs);
  g1.ldq = d;
  if ((err = traced("k1_gemm_mx8_resid_sumsq", gemm_flops(M, d, K),
                    (MK + Kd) * q8 + 2.0 * Md * e + Md * q8 + M * ws.Tn * 4.0 + d * e, s,
                    [&] { return coda::launch_gemm_mx8(g1, coda::EPI_RESID_SUMSQ, s); })) != hipSuccess)
    return hip_status(err);
  // M1: [g | u] = diag(r) (y gamma) W on MXFP8; epilogue r from the partial
  // sums, gu, a = silu(g) u (bf16) and a along F
  coda::MxQuantArgs qw{};
  qw.src = W;
  qw.ld = 2 * F;
  qw.rows = d;
  qw.cols = 2 * F;
  qw.qt = u8(ws.wq);
  qw.st = u8(ws.ws);
  qw.gated_F = F;
  if ((err = traced("x3_mx8_quantize_W_gateup", 0.0, 2.0 * dF * (e + q8), s,
                    [&] { return coda::launch_mx8_quantize_fused(qw, 0, s); })) != hipSuccess)
    return hip_status(err);
  GemmArgs m1 = gemm_mx8(M, F, d, u8(ws.ygq), u8(ws.ygs), u8(ws.wq), u8(ws.ws), gu, 2 * F);
  m1.B_total = (uint64_t)(2 * F * d);
  m1.B_bytes = (uint32_t)std::min<uint64_t>(m1.B_total, 0x7FFFFFF0ull);
  m1.sB_bytes = (uint32_t)(2 * F * (d / 32));
  m1.C2 = a;
  m1.ldc2 = F;
  m1.F = (int)F;
  m1.q_out = u8(ws.aq);
  m1.qs_out = u8(ws.as);
  m1.ldq = F;
  m1.part_row = P;
  m1.ld_part_row = ws.Tn;
  m1.nparts = ws.Tn;
  m1.inv_d = 1.0f / (float)d;
  m1.eps = eps;
  m1.r_out = r;
  if ((err = traced("m1_gemm_mx8_gateup_rsqrt_swiglu", gemm_flops(M, 2 * F, d),
                    (Md + 2.0 * dF) * q8 + 3.0 * MF * e + MF * q8 + M * ws.Tn * 4.0 + 4.0 * M, s,
                    [&] { return coda::launch_gemm_mx8(m1, coda::EPI_RSQRT_SWIGLU, s); })) != hipSuccess)
    return hip_status(err);
  // M2: z = a Wd on MXFP8
  if ((err = traced("x4_mx8_quantize_WdT", 0.0, dF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(Wd, d, F, d, u8(ws.wdq), u8(ws.wds), s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs m2 = gemm_mx8(M, d, F, u8(ws.aq), u8(ws.as), u8(ws.wdq), u8(ws.wds), z, d);
  return hip_status(traced("m2_gemm_mx8_down", gemm_flops(M, d, F), (MF + dF) * q8 + Md * e, s,
                           [&] { return coda::launch_gemm_mx8(m2, coda::EPI_STORE, s); }));
}

coda_status coda_mlp_bwd_mx8(int64_t M, int64_t K, int64_t d, int64_t F, const void* X, const void* W1,
                             const void* gamma, const void* W, const void* Wd, const void* y, const float* r,
                             const void* gu, const void* a, const void* dz, const void* dy_in, void* dX,
                             void* dW1, void* dR, void* dW, void* dWd, float* dgamma, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!X || !W1 || !gamma || !W || !Wd || !y || !r || !gu || !a || !dz || !dX || !dW1 || !dR || !dW || !dWd ||
      !dgamma)
    return CODA_ERR_NULL;
  if (!mlp_mx8_shape_ok(M, K, d, F)) return CODA_ERR_SHAPE;
  for (const void* p : {X, W1, gamma, W, Wd, y, (const void*)r, gu, a, dz, (const void*)dX, (const void*)dW1,
                        (const void*)dR, (const void*)dW, (const void*)dWd, (const void*)dgamma})
    if (!aligned16(p)) return CODA_ERR_ALIGN;
  if (dy_in && !aligned16(dy_in)) return CODA_ERR_ALIGN;
  const MlpMx8BwdWs ws = mlp_mx8_bwd_ws(M, K, d, F);
  if (!workspace || workspace_bytes < ws.total) return CODA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CODA_ERR_ALIGN;
  const size_t e = 2;
  const Range in[] = {rng(X, M * K * e), rng(W1, K * d * e), rng(gamma, d * e), rng(W, d * 2 * F * e),
                      rng(Wd, F * d * e), rng(y, M * d * e), rng(r, M * 4), rng(gu, M * 2 * F * e),
                      rng(a, M * F * e), rng(dz, M * d * e), rng(dy_in, dy_in ? M * d * e : 0)};
  const Range out[] = {rng(dX, M * K * e), rng(dW1, K * d * e), rng(dR, M * d * e), rng(dW, d * 2 * F * e),
                       rng(dWd, F * d * e), rng(dgamma, d * 4), rng(workspace, ws.total)};
  if (!alias_free(in, out)) return CODA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* wb = (char*)workspace;
  auto u8 = [&](size_t off) { return (uint8_t*)(wb + off); };
  hipError_t err;
  const double q8 = 1.0 + 1.0 / 32.0, Md = (double)M * d, dF = (double)d * F, MF = (double)M * F;
  // the SwiGLU part: dz along d and along M (one pass), Wd along d
  coda::MxQuantArgs qdz{};
  qdz.src = dz;
  qdz.ld = d;
  qdz.rows = M;
  qdz.cols = d;
  qdz.qr = u8(ws.dzq);
  qdz.sr = u8(ws.dzs);
  qdz.qt = u8(ws.dzTq);
  qdz.st = u8(ws.dzTs);
  if ((err = traced("w1_mx8_quantize_dz_both", 0.0, Md * (e + 2.0 * q8), s,
                    [&] { return coda::launch_mx8_quantize_fused(qdz, 0, s); })) != hipSuccess)
    return hip_status(err);
  if ((err = traced("w2_mx8_quantize_Wd", 0.0, dF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize(Wd, d, F, d, u8(ws.wdq), u8(ws.wds), s);
       })) != hipSuccess)
    return hip_status(err);
  // M3: da = dz Wd^T on MXFP8; epilogue dgu from the saved gu, quantised (as
  // bf16) along 2F and along M straight into the block part's dz operands
  char* blk = wb + ws.blk;
  GemmArgs m3 = gemm_mx8(M, F, d, u8(ws.dzq), u8(ws.dzs), u8(ws.wdq), u8(ws.wds), nullptr, 2 * F);
  m3.E = gu;
  m3.lde = 2 * F;
  m3.F = (int)F;
  m3.q_out = (uint8_t*)(blk + ws.b.dzq);
  m3.qs_out = (uint8_t*)(blk + ws.b.dzs);
  m3.ldq = 2 * F;
  m3.qt_out = (uint8_t*)(blk + ws.b.dzTq);
  m3.qts_out = (uint8_t*)(blk + ws.b.dzTs);
  m3.ldqt = M;
  if ((err = traced("m3_gemm_mx8_da_swiglu_bwd", gemm_flops(M, F, d), (Md + dF) * q8 + 2.0 * MF * e + 4.0 * MF * q8,
                    s, [&] { return coda::launch_gemm_mx8(m3, coda::EPI_SWIGLU_BWD, s); })) != hipSuccess)
    return hip_status(err);
  // M4: dWd = a^T dz on MXFP8: a along M, transposed
  if ((err = traced("w3_mx8_quantize_aT", 0.0, MF * (e + q8), s, [&] {
         return coda::launch_mx8_quantize_t(a, F, M, F, u8(ws.aTq), u8(ws.aTs), s);
       })) != hipSuccess)
    return hip_status(err);
  GemmArgs m4 = gemm_mx8(F, d, M, u8(ws.aTq), u8(ws.aTs), u8(ws.dzTq), u8(ws.dzTs), dWd, d);
  if ((err = traced("m4_gemm_mx8_dWd", gemm_flops(F, d, M), (MF + Md) * q8 + dF * e, s,
                    [&] { return coda::launch_gemm_mx8(m4, coda::EPI_STORE, s); })) != hipSuccess)
    return hip_status(err);
  // the block's MXFP8 backward with dz = dgu (its operands already made),
  // W2 = W (N = 2F) and dy_in
  return norm_bwd_mx8(M, K, d, 2 * F, X, W1, gamma, W, y, r, nullptr, dy_in, dX, dW1, dR, dW, dgamma, blk,
                      ws.b, s);
}

}  // extern "C"
