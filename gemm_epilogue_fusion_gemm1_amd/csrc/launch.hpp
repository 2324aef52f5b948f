// Internal interface between the C-ABI (api.cpp) and the kernels
// (kernels.hip).  Not installed; the public interface is include/coda.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

// Output tile of the MFMA GEMM kernels (bf16 and MXFP8) and of the fp32 fallback kernel.
// The partial-sum workspaces are laid out per tile, so the C-ABI sizes them
// from these constants.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileF32 = 64;

// Epilogue selector of the GEMM kernels.
enum Epi : int {
  EPI_STORE = 0,       // C = acc
  EPI_RESID_SUMSQ = 1, // y = acc + E; C = y; part_row[i][tile_n] = sum_{j in tile} y_ij^2;
                       // if C2: C2 = y * vcol (the RMSNorm weight, by column), stored
                       // transposed (C2[j][i], ldc2 = its row length) when c2_trans
  EPI_ROWSCALE = 2,    // C = vrow[i] * acc  (vrow NULL: vcol[i], bf16)
  EPI_DN = 3,          // dh = acc; C = dn = gamma_j dh; part_row = sum_j dn*y; part_col = sum_i dh*r*y;
                       // if C2: C2 = n = r_i y
  EPI_SWIGLU = 4,      // gate/up pair: C = gu (both halves), C2 = silu(g) * u
  EPI_SWIGLU_BWD = 5,  // da = acc; C = dgu from the saved gu in E
  EPI_RSQRT_SCALE = 6, // r_i = (sum_t part_row[i][t] * inv_d + eps)^-1/2; C = r_i acc;
                       // tiles of column 0 write r to r_out
  EPI_RSQRT_SWIGLU = 7,  // r_i as EPI_RSQRT_SCALE; gate/up pair scaled by r_i, then as
                         // EPI_SWIGLU: C = gu (both halves), C2 = silu(g) * u
  EPI_CE_STATS = 8,      // logits: C = acc; per row and tile: part_row = max_j acc,
                         // part_col = sum_j exp(acc - max) ([M][tiles_n] each, ld_part_row);
                         // lab_out[i] = acc[i][labels[i]] (written by the tile holding it)
  EPI_ROPE = 9,          // C = acc with the pairs (2i, 2i+1) of every rope_head-wide head in
                         // the first rope_rot columns rotated by the table's angle for
                         // position (row mod rope_seq)
};

// Operand layouts.  "K-major" = the contraction index is contiguous in memory.
struct GemmArgs {
  int M, N, K;                   // C is M x N (EPI_SWIGLU: N = F gate columns)
  const void* A; int64_t lda;    // A: M x K logical
  const void* B; int64_t ldb;    // B: K x N logical
  void* C; int64_t ldc;
  void* C2; int64_t ldc2;        // EPI_SWIGLU: a [M, F]
  const void* E; int64_t lde;    // epilogue matrix input: R (RESID), y (DN), gu (SWIGLU_BWD)
  const float* vrow;             // per-row vector: r (ROWSCALE in fwd, DN)
  const void* vcol;              // per-column / per-row vector in dtype: gamma
  float* part_row; int64_t ld_part_row;   // [M][tiles_n]
  float* part_col; int64_t ld_part_col;   // [tiles_m][N]
  int F;                         // SwiGLU half width (gate columns)
  int nparts; float inv_d; float eps; float* r_out;   // EPI_RSQRT_SCALE
  int c2_trans;                  // EPI_RESID_SUMSQ: C2 stored transposed
  const int* labels; float* lab_out;   // EPI_CE_STATS
  const float* rope_tab; int rope_rot, rope_head, rope_seq;   // EPI_ROPE: tab = [cos | sin],
                                                               // each [rope_seq][rope_head / 2]
  uint32_t A_bytes, B_bytes;     // operand extents when they fit one buffer (<= 2 GiB)
  // MXFP8 GEMMs (launch_gemm_mx8): A is [M][K] and B is given as B^T [N][K],
  // both E4M3 bytes with lda / ldb in bytes.  Their E8M0 scales are stored
  // step-blocked: [K/128][rows][4], the word of (step t, row r) holding the
  // scales of r's 32-blocks 4t..4t+3 (rows = M for A, N for B)
  const uint8_t* sA; const uint8_t* sB;
  uint32_t sA_bytes, sB_bytes;
  // EPI_RESID_SUMSQ in an MXFP8 GEMM: y * vcol quantised to MXFP8 along the
  // row, codes [M][ldq] and scales [ldq/128][M][4] (instead of C2)
  uint8_t* q_out; uint8_t* qs_out; int64_t ldq;
  // full operand extents; past 2 GiB the loaders reach an operand through
  // windows (a K-contiguous operand's 256 tile rows, an MN-contiguous
  // operand's K step)
  uint64_t A_total, B_total;
  // EPI_SWIGLU_BWD in an MXFP8 GEMM: dgu (as stored, bf16) quantised to MXFP8
  // along 2F into q_out / qs_out (ldq = 2F) and, when qt_out is set, along M
  // into qt_out [2F][ldqt] / qts_out [M/128][2F][4] (M % 128 == 0); C (the
  // bf16 dgu) may then be NULL
  uint8_t* qt_out; uint8_t* qts_out; int64_t ldqt;
};

// Launchers: enqueue on `stream`, return the hipGetLastError() after launch.
// a_kmajor / b_kmajor select the operand layouts; every epilogue is
// instantiated for the layout combinations the block uses.
hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_kmajor, bool b_kmajor, Epi epi,
                            hipStream_t stream);
hipError_t launch_gemm_f32(const GemmArgs& g, Epi epi, hipStream_t stream);
// MXFP8 x MXFP8 GEMM, both operands K-contiguous (A [M][K], B^T [N][K]);
// K % 128 == 0; epilogues EPI_STORE, EPI_RESID_SUMSQ (with q_out),
// EPI_RSQRT_SCALE, EPI_DN, EPI_ROWSCALE, EPI_SWIGLU and EPI_RSQRT_SWIGLU
// (B = the gate/up weight's 2F rows in gate/up order; a quantised into
// q_out along F), EPI_SWIGLU_BWD
hipError_t launch_gemm_mx8(const GemmArgs& g, Epi epi, hipStream_t stream);
// codes / scales = the MXFP8 quantisation of src [rows, cols] (bf16, row
// stride ld) along its rows, stored transposed: codes [cols][rows], scales
// step-blocked [rows/128][cols][4] (rows % 128 == 0, cols % 8 == 0)
hipError_t launch_mx8_quantize_t(const void* src, int64_t ld, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream);
// codes / scales = the MXFP8 quantisation of the bf16 rows of src along the
// row (cols % 128 == 0; codes [rows][cols], scales step-blocked
// [cols/128][rows][4])
hipError_t launch_mx8_quantize(const void* src, int64_t ld, int64_t rows, int64_t cols,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream);

// One pass over a bf16 [rows, cols] tensor (row stride ld) that makes MXFP8
// operands of the backward (rows % 128 == 0).  mode 0: v = src; mode 1: v =
// dy = r_i src - c_i y (+ dy_in unless NULL), rounded to bf16 and written to
// out (out may be src);
// mode 2: v = r_i src rounded to bf16.  qr / sr: v quantised along the row
// (codes [rows][cols], scales step-blocked [cols/128][rows][4]; cols % 128 ==
// 0; not made in mode 2); qt / st: v quantised along the column, stored
// transposed (codes [cols][rows], scales [rows/128][cols][4]).  qr NULL: no
// row-wise codes.  gated_F > 0: src is a gate/up weight [d, 2F] and its
// column c is written to transposed row 64 (j / 32) + 32 [c >= F] + j % 32,
// j = c mod F: each 64-row group holds 32 gate rows and the 32 up rows of the
// same j, the column order of a gate/up GEMM's tile (F % 32 == 0).
struct MxQuantArgs {
  const void* src; int64_t ld;
  int64_t rows, cols;
  const float* r; const float* c; const void* y; const void* dy_in; void* out;
  uint8_t* qr; uint8_t* sr;
  uint8_t* qt; uint8_t* st;
  int64_t gated_F;
};
hipError_t launch_mx8_quantize_fused(const MxQuantArgs& q, int mode, hipStream_t stream);

// r[i] = (sum_t P[i][t] / d + eps)^(-1/2)
hipError_t launch_row_rsqrt(const float* P, int64_t ldp, int T, int64_t M, int64_t d, float eps,
                            float* r, hipStream_t stream);
// c[i] = r_i^3 * (sum_t S[i][t]) / d ;  dgamma[j] = sum_tau G[tau][j]
hipError_t launch_bwd_reduce(const float* S, int64_t lds, int Tn, const float* r, int64_t M,
                             int64_t d, const float* G, int Tm, float* c, float* dgamma,
                             hipStream_t stream);
// tab[p][i] = cos(p base^(-2i/D)), tab[S*D/2 + p*D/2 + i] = sin(...), computed in
// double and stored as float; p < S, i < D/2
hipError_t launch_rope_table(float* tab, int S, int D, double base, hipStream_t stream);
// dP = the pairs of dY's first N_rot columns rotated back by -angle (the
// transpose of the forward rotation); the other columns copied (bf16)
hipError_t launch_rope_inverse(const void* dY, const float* tab, void* dP, int64_t M, int64_t N,
                               int N_rot, int D, int S, hipStream_t stream);
// lse[i] = m + log s over the tiles' (max, sum-exp) pairs combined in order;
// loss[i] = lse[i] - lab[i], or 0 when labels[i] lies outside [0, V)
hipError_t launch_ce_combine(const float* pmax, const float* psum, int64_t ldp, int T,
                             const float* lab, const int* labels, int64_t V, int64_t M, float* lse,
                             float* loss, hipStream_t stream);
// dlogits[i][j] = dloss[i] (exp(logits[i][j] - lse[i]) - [j == labels[i]])  (bf16);
// 0 for a row whose label lies outside [0, V)
hipError_t launch_ce_dlogits(const void* logits, const int* labels, const float* lse,
                             const float* dloss, void* dlogits, int64_t M, int64_t V,
                             hipStream_t stream);
// in place: dR[i][j] = r_i dR[i][j] - c_i y[i][j] (+ dy_in[i][j] when dy_in is
// not NULL)  (dR holds dn on entry)
hipError_t launch_dy(void* dR, const void* y, const float* r, const float* c, const void* dy_in,
                     int64_t M, int64_t d, hipStream_t stream);

// Size of the built-in device scratch of coda_fwd_noalloc (80 MiB: the
// forward workspace of the LLaMA-7B- and 70B-hidden-shaped blocks fits).
constexpr size_t kNoAllocScratchBytes = (size_t)80 << 20;
// The current device's copy of that scratch (its address is looked up on the
// first call on each device and kept); no allocation.
hipError_t noalloc_scratch(void** ptr);

}  // namespace coda
