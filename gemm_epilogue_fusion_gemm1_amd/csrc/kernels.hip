// HIP kernels of the fused GEMM-Residual-RMSNorm-GEMM block and the SwiGLU
// block for CDNA4 (gfx950).
//
// The method (CODA, "Rewriting Transformer Blocks as GEMM-Epilogue Programs",
// as reported by the toolin.ai blog section 核心の洞察 and the kucoin.com
// news flashes, sections "CODA: В «Финале» спрятаны сокровища" and
// "CODA : « La fin » cache un trésor"): a GEMM is a tiled multiply-accumulate
// main loop plus an epilogue that runs while the output tile is still in
// registers; memory-bound neighbours of a GEMM (residual add, the RMS row
// scale, SwiGLU) are rewritten to run inside that epilogue.  Here:
//
//  * one MFMA main loop for bf16 (v_mfma_f32_16x16x32_bf16) and MXFP8
//    (v_mfma_scale_f32_32x32x64_f8f6f4), fp32 accumulators, 256x256 output
//    tile per 512-thread workgroup, 8 waves of 128x64 (two per SIMD), a ring
//    of two or four LDS stages filled by direct-to-LDS loads;
//  * operand tiles are staged in LDS in the layout they have in memory,
//    with 16-byte chunks XOR-swizzled so that every LDS access of the loop
//    is free of bank conflicts on gfx950's 64-bank LDS (16 lanes x 16 bytes
//    per cycle).  A tile whose contraction index is contiguous is read as
//    MFMA fragments with ds_read_b128; a tile whose MN index is contiguous is
//    read with two ds_read_b64_tr_b16 (transpose reads) per fragment, so no
//    operand is ever transposed in registers;
//  * epilogues selected at compile time (launch.hpp: Epi) work on the
//    accumulator registers in place: residual add + per-tile partial sums of
//    squares, row scale, the RMSNorm-backward epilogue, SwiGLU and its
//    backward.  The epilogue moves the accumulators through LDS into a
//    row-major assignment (16-byte global accesses, row sums in 3 lane
//    shuffles); waves that share rows or columns combine through LDS in a
//    fixed order, so every result is run-to-run deterministic (no atomics).
#include "launch.hpp"

#include <mutex>
#include <type_traits>

namespace coda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = kTileM;
constexpr int BN = kTileN;
constexpr uint32_t OOB = 0x80000000u;            // voffset past every extent -> loads 0

// K step and depth of the LDS ring of one GEMM instantiation.  K-contiguous
// operands want 128-byte row segments (K step 64, two stages); when both
// operands are MN-contiguous a K step of 32 with a four-stage ring hides more
// load latency.  Both fill 128 KiB of LDS.
template <int BKv, int NSTv>
struct KCfg {
  static constexpr int BK = BKv;                       // K step
  static constexpr int NSTAGE = NSTv;                  // LDS ring of K steps
  static constexpr int OPER_BYTES = BM * BK * 2;       // one operand tile, unpadded
  static constexpr int STAGE_BYTES = 2 * OPER_BYTES;   // A + B
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  static constexpr int KROW = BK * 2;                  // bytes of one K-contiguous tile row
  static constexpr int KCH = BK / 8;                   // 16-byte chunks per such row
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(NSTAGE >= 2 && LDS_BYTES <= 160 * 1024, "LDS ring");
  static_assert(LDS_BYTES >= 8 * 8192 + 6144, "epilogue staging fits in the ring");
  // K-contiguous tile: row m at m*KROW, chunk q at position q ^ kswz(m); the
  // position changes every two rows
  static __device__ __forceinline__ int kswz(int m) { return (m >> 1) % KCH; }
  static __device__ __forceinline__ int kmaj_off(int m, int q) {
    return m * KROW + ((q ^ kswz(m)) << 4);
  }
};
static_assert(BM == BN, "operand tiles share one LDS geometry");

// LDS tile layouts (256 MN x 32 K, bf16):
// (BK = K step; see KCfg)
//  K-contiguous:  row m (2 BK bytes) at m*2BK; its 16-byte k chunk q (k =
//                 8q..8q+7) sits at chunk position q ^ ((m / 2) % KCH).  The
//                 16 lanes that read chunk q of rows m..m+15 (m % 16 == 0)
//                 are then free of bank conflicts for 128- and 64-byte rows
//                 (measured with rocprofv3's LDS bank-conflict counter; with
//                 64-byte rows a position that changed every four rows, one
//                 256-byte bank line, conflicted 2-way).
//  MN-contiguous: row k (512 B) at k*512; its 16-byte MN chunk c (mn =
//                 8c..8c+7) sits at chunk position c ^ mn_swz(k), mn_swz(k) =
//                 ((k & 3) << 2) | (((k >> 3) & 1) << 1).  A transpose read
//                 of 32 lanes touches either 4 rows x 4 chunks (32-wide
//                 blocks) or, for 16-wide blocks, 4 rows x 2 chunks in each of
//                 two row groups 8 apart; the swizzle spreads both over all 16
//                 bank groups (the k bit 3 term separates the two groups).
// Both are filled by direct-to-LDS buffer loads: one 64-lane load writes 1 KiB
// of contiguous LDS (lane l at +16 l), so the swizzle is applied by choosing
// which global chunk each lane fetches.
__device__ __forceinline__ int mn_swz(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 1); }
__device__ __forceinline__ int mnmaj_off(int k, int c) { return k * 512 + ((c ^ mn_swz(k)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer: stride 0, num_records in bytes; dword3 0x00020000 = 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// A buffer that starts `off` bytes into a tensor of `total` bytes.  Offsets
// within it are 32-bit and OOB (2^31) must lie past its end, so it covers at
// most kMaxWindow bytes; a tensor larger than that is reached through windows
// based nearer the data (a tile's first row, a K step's first row).
constexpr uint64_t kMaxWindow = 0x7FFFFFF0ull;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window_rsrc(const void* p, uint64_t total, uint64_t off) {
  const uint64_t left = off < total ? total - off : 0;
  return make_rsrc((const char*)p + off, (uint32_t)(left < kMaxWindow ? left : kMaxWindow));
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

__device__ __forceinline__ float bf2f(__bf16 h) { return (float)h; }
__device__ __forceinline__ __bf16 f2bf(float f) { return (__bf16)f; }  // round to nearest even

// Tile id -> (tile_m, tile_n).  Workgroups are dealt round-robin over the 8
// XCDs (wg % 8), each with its own L2; consecutive logical tiles are given to
// one XCD so that the tiles resident on an XCD share operand rows/columns.
// Within that order, groups of GM tile-rows are walked column by column.
#ifndef CODA_TILE_GROUP_M
#define CODA_TILE_GROUP_M 8
#endif
#ifndef CODA_XCD_REMAP
#define CODA_XCD_REMAP 1
#endif
#ifndef CODA_BF16_MFMA16
#define CODA_BF16_MFMA16 1
#endif
// Two-stage main loops: issue a stage's loads right after the previous
// step's barrier instead of at the start of the step before its use
// (MXFP8, and the bf16 loop with 64-k steps)
#ifndef CODA_MX_EARLY_ISSUE
#define CODA_MX_EARLY_ISSUE 1
#endif
#ifndef CODA_BF16_EARLY_ISSUE
#define CODA_BF16_EARLY_ISSUE 1
#endif
// Waves that issue the operand tiles' direct-to-LDS loads.  Waves w and w + 4
// share a SIMD.  A wave issuing a burst of loads stalls at each issue.  When
// all 8 waves load right after the barrier, both waves of every SIMD stall
// together and its MFMA pipe idles.  With waves 0-3 issuing twice the loads
// and waves 4-7 none, each SIMD has one wave free to issue MFMAs meanwhile.
// In an in-bounds probe of this loop (two sub-steps of 12 LDS reads and 32
// MFMAs per wave, L2-resident operands), MFMA utilisation went from 72% with
// 8 loading waves to 86% with 4.
// Measured per GEMM on the LLaMA-7B/70B and SwiGLU steps: 4 loading waves
// are 1.5-7.5% faster for the bf16 GEMMs (every layout, with the K-step /
// ring choice below) and 1-3% slower for MXFP8, which keeps all 8.
#ifndef CODA_LOAD_WAVES
#define CODA_LOAD_WAVES 4
#endif
#ifndef CODA_MX_LOAD_WAVES
#define CODA_MX_LOAD_WAVES 8
#endif
static_assert((CODA_LOAD_WAVES == 4 || CODA_LOAD_WAVES == 8) && (CODA_MX_LOAD_WAVES == 4 || CODA_MX_LOAD_WAVES == 8),
              "loading waves: 4 (one per SIMD) or all 8");
__device__ __forceinline__ void map_tile(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int t = wg;
  if (CODA_XCD_REMAP) {
    const int q = total >> 3, rem = total & 7;
    const int x = wg & 7, i = wg >> 3;
    t = (x < rem) ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
  }
  constexpr int GM = CODA_TILE_GROUP_M;
  const int group = GM * tiles_n;
  const int gidx = t / group;
  const int first_m = gidx * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in = t - gidx * group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// ---------------------------------------------------------------------------
// Workgroup shape.  A GEMM workgroup computes a BM x BN output tile with a
// WM x WN grid of waves; each wave owns a TM x TN sub-tile made of FM x FN
// 32x32 MFMA blocks.  With 8 waves (2 x 4) two waves share each SIMD, so one
// wave's waits (LDS, global loads, the per-step barrier) are covered by the
// other wave's MFMAs.
// ---------------------------------------------------------------------------
template <int WM_, int WN_>
struct Grid {
  static constexpr int WM = WM_, WN = WN_, NT = 64 * WM_ * WN_;
  static constexpr int TM = BM / WM_, TN = BN / WN_;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
};

// ---------------------------------------------------------------------------
// Operand staging: buffer loads straight into LDS (no register staging).
// Out-of-range chunks get an out-of-range offset and land as zeros, so edge
// tiles and K tails need no branch.  Each wave fills LP KiB per operand tile.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;

// One 64-lane direct-to-LDS load: lane l's 16 bytes at global `voff` land at
// LDS byte `dst` + 16 l (dst is wave-uniform and goes through M0).  It is
// issued from inline assembly so that the compiler does not track it as a
// pending LDS write: the kernel itself waits (s_waitcnt vmcnt) and synchronises
// (barrier) before any wave reads the stage it fills, and otherwise the
// compiler would make every LDS read of the loop wait for all such loads.  No
// other code in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, lds_char* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(m0)
               : "memory", "m0");
}
// The same for 4 bytes per lane: lane l's dword lands at `dst` + 4 l.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, lds_char* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Contraction index contiguous: the matrix is [MN rows][K], reached through a
// buffer based at the tile's first row.  Load p of wave w
// fills the 1 KiB of tile rows R(LP w + p) .. +R-1 (R = 1024 / 2BK): lane l
// takes row +l/KCH and the k chunk whose swizzled position is l%KCH.  The
// swizzle repeats every two loads, so a lane keeps one base offset and one
// chunk per load parity and derives the rest.
template <class KC, int NT, bool GATED, bool WIN>
struct LoaderKMajor {
  static constexpr int LP = KC::OPER_BYTES / 1024 / (NT / 64);
  static constexpr int R = 1024 / KC::KROW;       // tile rows per load
  static_assert(LP % 2 == 0 && R % KC::KCH == 0, "swizzle period");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t gbase[2];    // byte offset of the lane's row and chunk at k0 = 0 (loads 0 and 1)
  int kq[2];            // k offset of the lane's chunk (even / odd loads)
  int row;              // the lane's row in load 0, minus the row count
  uint32_t pair;        // bytes between loads p and p + 2
  int K;
  int ldsoff;           // wave's first byte within an operand tile

  __device__ void init(const void* ptr, uint64_t bytes, int64_t ld, int row0, int rows, int K_,
                       int t, int, int) {
    // WIN: the buffer starts at the tile's first row, so offsets stay below
    // 256 rows; else it covers the whole matrix (at most 2 GiB)
    const uint32_t ldb = (uint32_t)(ld * 2);
    rs = WIN ? window_rsrc(ptr, bytes, (uint64_t)row0 * ldb) : make_rsrc(ptr, (uint32_t)bytes);
    K = K_;
    const int w = t >> 6, l = t & 63;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int m = R * (LP * w + p) + l / KC::KCH;
      const int q = (l % KC::KCH) ^ KC::kswz(m);
      kq[p] = 8 * q;
      gbase[p] = (uint32_t)(WIN ? m : row0 + m) * ldb + (uint32_t)(16 * q);
    }
    row = row0 + R * LP * w + l / KC::KCH - rows;
    pair = 2u * R * ldb;
    ldsoff = __builtin_amdgcn_readfirstlane(w) * LP * 1024;
  }
  __device__ void issue_one(lds_char* tile, int k0, int p) const {
    const bool ok = (row + R * p) < 0 && (k0 + kq[p & 1]) < K;
    dma16(rs, ok ? gbase[p & 1] + (uint32_t)(p >> 1) * pair + (uint32_t)(k0 * 2) : OOB,
          tile + ldsoff + p * 1024);
  }
  __device__ void issue(lds_char* tile, int k0) const {
#pragma unroll
    for (int p = 0; p < LP; ++p) issue_one(tile, k0, p);
  }
};

// Contraction index strided: the matrix is [K rows][MN cols], reached
// through a buffer based at each K step's first row.  Load p of
// wave w fills tile k rows 2(LP w + p) and +1: lane l takes row +l/32 and the
// MN chunk whose swizzled position is l%32.  The swizzle of row k depends on
// k % 4 and bit 3 of k, so the chunk a lane fetches repeats with the load's
// phase: its parity, and (when a wave fills more than 8 k rows) which half
// of each 16-row block it falls in.  GATED maps tile columns onto the [gate |
// up] halves of a [d, 2F] weight: the tile is cut into groups of TN columns
// (one 64-column epilogue half) whose first half holds gate columns j and
// second half the up columns F + j of the same j, so one lane ends up holding
// a gate and its up value.
template <class KC, int NT, bool GATED, int TN, bool WIN>
struct LoaderMNMajor {
  static constexpr int LP = KC::OPER_BYTES / 1024 / (NT / 64);
  static_assert(LP % 2 == 0 && (LP <= 4 || LP % 8 == 0), "swizzle period");
  static constexpr int NPH = LP >= 8 ? 4 : 2;   // load phases with distinct chunks
  // phase of load p: its parity, and bit 2 of (LP w + p) = bit 3 of its k row
  // (LP w is a multiple of 8 when LP >= 8, so p alone decides it)
  static __device__ __forceinline__ constexpr int phase(int p) { return (p & 1) | (NPH == 4 ? ((p >> 2) & 1) << 1 : 0); }
  // first load of phase ph
  static __device__ __forceinline__ constexpr int first(int ph) { return (ph & 1) | ((ph >> 1) << 2); }
  __amdgpu_buffer_rsrc_t rs;     // one buffer over the whole matrix (at most 2 GiB) ...
  const char* base;              // ... or (WIN) the matrix, read through a buffer
                                 // based at each K step's first row
  uint32_t gbase[NPH];  // the first load of each phase, at k0 = 0
  bool colok[NPH];
  int krow;             // the lane's k row in load 0, minus K
  uint32_t ldb;
  int ldsoff;

  __device__ void init(const void* ptr, uint64_t bytes, int64_t ld, int col0, int cols, int K_,
                       int t, int F, int tn) {
    if constexpr (WIN) base = (const char*)ptr;
    else rs = make_rsrc(ptr, (uint32_t)bytes);
    ldb = (uint32_t)(ld * 2);
    const int w = t >> 6, l = t & 63;
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      const int p = first(ph);
      const int k = 2 * (LP * w + p) + (l >> 5);
      const int c = (l & 31) ^ mn_swz(k);   // the same for every load of this phase
      int col;
      bool ok;
      if (GATED) {
        constexpr int GH = TN / 2;
        const int lc = c * 8;                     // tile column 0..255
        const int grp = lc / TN, sub = lc % TN;
        const int j = tn * (BN / 2) + grp * GH + (sub % GH);
        ok = j < F;
        col = (sub < GH) ? j : F + j;
      } else {
        col = col0 + c * 8;
        ok = col < cols;
      }
      colok[ph] = ok;
      gbase[ph] = (uint32_t)k * ldb + (uint32_t)col * 2u;
    }
    krow = 2 * LP * w + (l >> 5) - K_;
    ldsoff = __builtin_amdgcn_readfirstlane(w) * LP * 1024;
  }
  __device__ void issue_one(lds_char* tile, int k0, int p) const {
    const int ph = phase(p);
    const bool ok = colok[ph] && (k0 + krow + 2 * p) < 0;
    // load p's k row is that of its phase's first load plus 2 (p - first)
    dma16(rs, ok ? gbase[ph] + (uint32_t)(k0 + 2 * (p - first(ph))) * ldb : OOB,
          tile + ldsoff + p * 1024);
  }
  __device__ void issue(lds_char* tile, int k0) const {
    if constexpr (WIN) {
      // The window starts at the step's first row and spans the largest
      // 32-bit range below OOB.  Every lane whose row or column lies outside
      // the matrix is sent to OOB by its own check, so the window's end never
      // has to match the matrix's: scalar arithmetic only, no branch.
      const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (uint64_t)(uint32_t)k0 * ldb, (uint32_t)kMaxWindow);
#pragma unroll
      for (int p = 0; p < LP; ++p) {
        const int ph = phase(p);
        const bool ok = colok[ph] && (k0 + krow + 2 * p) < 0;
        dma16(r, ok ? gbase[ph] + (uint32_t)(2 * (p - first(ph))) * ldb : OOB, tile + ldsoff + p * 1024);
      }
    } else {
#pragma unroll
      for (int p = 0; p < LP; ++p) issue_one(tile, k0, p);
    }
  }
};

template <bool KMAJ, class KC, int NT, bool GATED, int TN, bool WIN>
struct LoaderSel;
template <class KC, int NT, bool GATED, int TN, bool WIN>
struct LoaderSel<true, KC, NT, GATED, TN, WIN> { using type = LoaderKMajor<KC, NT, GATED, WIN>; };
template <class KC, int NT, bool GATED, int TN, bool WIN>
struct LoaderSel<false, KC, NT, GATED, TN, WIN> { using type = LoaderMNMajor<KC, NT, GATED, TN, WIN>; };

// bf16 MFMA operand fragments: 8 k values of one row (or column) of a
// 16- or 32-wide block per lane (see the readers below).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <bool KMAJ, class KC, int NB, int MBK>
struct FragReader;

// MXFP8 operand fragments of v_mfma_scale_f32_32x32x64_f8f6f4 (measured with
// an in-bounds probe): lane l supplies row (or column) l%32 of a 32-wide block
// and 32 E4M3 bytes of the sub-step's 64 k: bytes 0..15 from the first
// 32-block of k, bytes 16..31 from the second, each the 16 k values 16(l/32)
// .. +15 of that block.  Its scale operand covers (row l%32, k block l/32).
// The tile is K-contiguous in LDS with the bf16 geometry (128-byte rows, one
// row per 128 k), so the two halves are 16-byte chunks 4s + l/32 and
// 4s + 2 + l/32 of sub-step s, read with ds_read_b128 each.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
template <class KC>
struct FragReaderMX {
  int off0[2], off1[2];   // per sub-step s, for block 0; block i adds 32 rows
  __device__ void init(int mn0, int lane) {
    const int l32 = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      off0[s] = KC::kmaj_off(mn0 + l32, 4 * s + khalf);
      off1[s] = KC::kmaj_off(mn0 + l32, 4 * s + 2 + khalf);
    }
  }
  __device__ i32x8 read(const char* tile, int s, int i) const {
    const i32x4 lo = *(const i32x4*)(tile + off0[s] + i * 32 * KC::KROW);
    const i32x4 hi = *(const i32x4*)(tile + off1[s] + i * 32 * KC::KROW);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// K-contiguous tile: one ds_read_b128 per fragment.  32-row blocks
// (v_mfma_f32_32x32x16_bf16): lane l takes row l%32 and the 8 k 16s +
// 8(l/32)..+7 of sub-step s (16 k); 16-row blocks (v_mfma_f32_16x16x32_bf16):
// row l%16 and the 8 k 32s + 8(l/16)..+7 of sub-step s (32 k).  A and B are
// read with the same k assignment, which is all the product needs.
template <class KC, int NB, int MBK>
struct FragReader<true, KC, NB, MBK> {
  static constexpr int SUBK = MBK == 32 ? 16 : 32;   // k per sub-step
  int off[KC::BK / SUBK];   // per sub-step s, for block 0; block i adds MBK rows
  __device__ void init(int mn0, int lane) {
    const int r = lane % MBK, kq = lane / MBK;
#pragma unroll
    for (int s = 0; s < KC::BK / SUBK; ++s) off[s] = KC::kmaj_off(mn0 + r, (SUBK / 8) * s + kq);
  }
  __device__ bf16x8 read(const char* tile, int s, int i) const {
    return *(const bf16x8*)(tile + off[s] + i * MBK * KC::KROW);
  }
};

// MN-contiguous tile: two transpose reads per fragment.  Within a 16-lane
// group, ds_read_b64_tr_b16 hands output lane i element i%4 of the 8 bytes
// addressed by source lanes 4k + i/4 (k = 0..3).  Source lane j points at
// (k row K0 + j/4, columns c0 + 4(j%4)..+3), so output lane i receives
// column c0 + i at rows K0..K0+3.  32-column blocks: lanes 16..31 take
// columns +16 and lanes 32..63 k rows +8; 16-column blocks: the four 16-lane
// groups take k rows +0, +8, +16, +24.
template <class KC, int NB, int MBK>
struct FragReader<false, KC, NB, MBK> {
  static constexpr int SUBK = MBK == 32 ? 16 : 32;   // k rows per sub-step
  int off[NB];  // per block i; sub-step s and half h add k rows
  __device__ void init(int mn0, int lane) {
    const int j = lane & 15;
    const int krow = (MBK == 32 ? 8 * (lane >> 5) : 8 * (lane >> 4)) + (j >> 2);   // + SUBK s + 4 h
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int mn = mn0 + i * MBK + (MBK == 32 ? (lane & 16) : 0) + 4 * (j & 3);
      off[i] = mnmaj_off(krow, mn >> 3) + ((mn & 7) << 1);  // mn_swz(krow + SUBK s + 4h) == mn_swz(krow)
    }
  }
  __device__ bf16x8 read(const char* tile, int s, int i) const {
    const char* p = tile + off[i] + s * SUBK * 512;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// ---------------------------------------------------------------------------
// Epilogue helpers
// ---------------------------------------------------------------------------

// Accumulator layout.  The MFMA is issued with the B fragment as its first
// operand and the A fragment as its second, so it accumulates C^T blocks.
// 32x32 blocks: lane l, register r of block (i, j) holds C[row = 32i + l%32]
// [col = 32j + 8(r/4) + 4(l/32) + r%4]; 16x16 blocks: register r of block
// (i, j) holds C[16i + l%16][16j + 4(l/16) + r].  A lane thus owns one row
// and, per group of four registers, four consecutive columns, which the
// epilogue writes to LDS as 16-byte vectors.
__device__ __forceinline__ f32x4 quad(const f32x16& a, int g) {
  return f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoid_f(float g) { return 1.0f / (1.0f + __expf(-g)); }

// Lanes of one wave hand data to each other through LDS in the epilogue.  The
// compiler treats the lanes as separate threads, so without this it may move
// one lane's LDS write past another lane's read of the same bytes (a variant
// of the tile loop did: with part of a wave masked off, the next pass's
// writes were duplicated into the masked-off lanes' path, which ran before
// the other lanes' reads).  A convergent wave barrier between two fences
// pins the order; no instruction is emitted for it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// The MFMA GEMM: C[M,N] = A[M,K] B[K,N] (+ epilogue EPI), operands in bf16
// (FMT_BF16) or MXFP8 (FMT_MX8: E4M3 with an E8M0 scale per 32 k, both
// operands K-contiguous, A [M][K] and B^T [N][K]).  One body serves both:
// only the main loop differs.
// ---------------------------------------------------------------------------
enum Fmt : int { FMT_BF16 = 0, FMT_MX8 = 1 };

// x scaled into the E4M3 range and saturated at +-448 for the conversion; a
// NaN or an infinity passes through (fminf / fmaxf would turn a NaN into a
// finite bound), so the conversion makes it the NaN code and it propagates
// through the GEMMs instead of vanishing.  Finite values are unchanged.
__device__ __forceinline__ float mx8_sat(float x, float inv) {
  const float v = x * inv;
  return __builtin_isfinite(v) ? fminf(fmaxf(v, -448.0f), 448.0f) : v;
}

// One 32-block held by one lane to MXFP8: its 32 codes packed four to a
// word (w[j] holds elements 4j..4j+3), the shared exponent returned.  Same
// arithmetic as the 4-lane routine below.
__device__ __forceinline__ int mx8_block32(const float (&v)[32], uint32_t (&w)[8]) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(v[e]));
  const int sexp = max((int)((__float_as_uint(am) >> 23) & 255) - 135, -127);
  const float inv = __uint_as_float((uint32_t)(127 - sexp) << 23);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(mx8_sat(v[4 * j], inv), mx8_sat(v[4 * j + 1], inv), 0, false);
    w[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(mx8_sat(v[4 * j + 2], inv), mx8_sat(v[4 * j + 3], inv), x,
                                                     true);
  }
  return sexp;
}

// One 32-block of a row to MXFP8, shared by 4 consecutive lanes holding 8
// values each (lanes 4j..4j+3 of the wave): the block maximum by two
// shuffles, the shared exponent floor(log2 amax) - 8 (clamped at -127) from
// its exponent field, the 8 values scaled by the exact power of two,
// saturated at 448 and rounded to nearest even by the hardware conversion.
// Returns the lane's 8 codes; `sexp` receives the exponent.
__device__ __forceinline__ uint2 mx8_block_of_4_lanes(f32x4 lo, f32x4 hi, int& sexp) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) am = fmaxf(am, fmaxf(fabsf(lo[e]), fabsf(hi[e])));
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  sexp = max((int)((__float_as_uint(am) >> 23) & 255) - 135, -127);
  const float inv = __uint_as_float((uint32_t)(127 - sexp) << 23);
  auto sat = [&](float v) { return mx8_sat(v, inv); };
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(lo[0]), sat(lo[1]), 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(lo[2]), sat(lo[3]), w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(hi[0]), sat(hi[1]), 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(hi[2]), sat(hi[3]), w1, true);
  return uint2{(uint32_t)w0, (uint32_t)w1};
}


template <int FMT, int WMv, int WNv, int BKv, int NSTv, bool AK, bool BKM, int EPI, bool WIN>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
  using G = Grid<WMv, WNv>;
  using KC = KCfg<BKv, NSTv>;
  constexpr int FM = G::FM, FN = G::FN, TM = G::TM, TN = G::TN;
  constexpr int BK = KC::BK, NSTAGE = KC::NSTAGE, OPER_BYTES = KC::OPER_BYTES;
  constexpr int STAGE_BYTES = KC::STAGE_BYTES;
  // MXFP8: the ring holds E4M3 tiles in the bf16 geometry (a 128-byte row is
  // 128 k, so one K step of BK bf16 "units" is 2 BK k); each stage's scales,
  // BM + BN rows x 4 bytes (the step's four 32-blocks), follow the ring
  constexpr int SC_STAGE = (BM + BN) * 4;
  constexpr int SMEM_BYTES = KC::LDS_BYTES + (FMT == FMT_MX8 ? NSTAGE * SC_STAGE : 0);
  static_assert(FMT == FMT_BF16 || (AK && BKM && BK == 64), "MXFP8 operands are K-contiguous");
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  constexpr bool GATED = (EPI == EPI_SWIGLU || EPI == EPI_RSQRT_SWIGLU);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6, wm = wave / WNv, wn = wave % WNv;

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = GATED ? (g.N + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  int tm, tn;
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * BM, col0 = tn * BN;

  // the loaders split each operand tile over the loading waves (64 threads each)
  constexpr int LNT = (FMT == FMT_MX8 ? CODA_MX_LOAD_WAVES : CODA_LOAD_WAVES) * 64;
  static_assert(LNT <= G::NT, "loading waves");
  typename LoaderSel<AK, KC, LNT, false, TN, WIN>::type la;
  typename LoaderSel<BKM, KC, LNT, GATED, 64, WIN>::type lb;   // gate/up groups of one 64-column half
  // MXFP8: the loaders count in 2-byte units (K / 2, ld / 2)
  constexpr int U = FMT == FMT_MX8 ? 2 : 1;
  la.init(g.A, WIN ? g.A_total : g.A_bytes, g.lda / U, row0, g.M, g.K / U, t, 0, tm);
  // rows of the B operand: N, or for a gate/up GEMM on MXFP8 the 2F rows of
  // the weight stored with each 64-row group holding 32 gate rows j and the
  // 32 up rows of the same j (the order a gated tile's columns take), so that
  // the plain K-contiguous loader reads a gated tile as rows col0..col0+255
  const int nb = (FMT == FMT_MX8 && GATED) ? 2 * g.F : g.N;
  lb.init(g.B, WIN ? g.B_total : g.B_bytes, g.ldb / U, col0, nb, g.K / U, t, g.F, tn);

  // MFMA blocks: bf16 uses v_mfma_f32_16x16x32_bf16 (16x16 blocks, four
  // accumulators per lane), which draws less power per flop than the 32x32
  // form and so sustains a higher clock under the power limit; MXFP8 uses
  // v_mfma_scale_f32_32x32x64_f8f6f4 (32x32 blocks, sixteen per lane).
  constexpr int MB = (FMT == FMT_BF16 && CODA_BF16_MFMA16) ? 16 : 32;
  constexpr int BFM = TM / MB, BFN = TN / MB;
  using AccV = std::conditional_t<MB == 16, f32x4, f32x16>;
  AccV acc[BFM][BFN];
#pragma unroll
  for (int i = 0; i < BFM; ++i)
#pragma unroll
    for (int j = 0; j < BFN; ++j) acc[i][j] = AccV{};

  const int nk = (g.K / U + BK - 1) / BK;
  lds_char* lsm = (lds_char*)smem;
  constexpr int LPW = OPER_BYTES / 1024 / (LNT / 64) * 2;     // loads per loading wave per step
  constexpr int VM_NEXT = (NSTAGE - 2) * LPW;                 // loads allowed in flight
  static_assert(VM_NEXT < 64, "vmcnt range");
  static_assert(FMT == FMT_BF16 || VM_NEXT == 0, "MXFP8 waits for every load of the next step");
  // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 (7 and 15 = no wait)
  constexpr int WAIT_NEXT = (VM_NEXT & 15) | ((VM_NEXT >> 4) << 14) | (7 << 4) | (15 << 8);
  const bool loader = __builtin_amdgcn_readfirstlane(wave) < LNT / 64;   // wave-uniform
  auto issue = [&](int step) {
    lds_char* st = lsm + (step % NSTAGE) * STAGE_BYTES;
    if constexpr (LNT == G::NT) {
      la.issue(st, step * BK);
      lb.issue(st + OPER_BYTES, step * BK);
    } else if (loader) {
      la.issue(st, step * BK);
      lb.issue(st + OPER_BYTES, step * BK);
    }
  };

  if constexpr (FMT == FMT_MX8) {
    static_assert(WMv * WNv == 8, "the MXFP8 scale staging assumes 8 waves");
    // Same pipeline as the bf16 loop below (two sub-steps of 64 k per K step
    // of 128), plus the scales: each wave loads 64 rows' 4 scale bytes of the
    // step (waves 0-3 A rows, 4-7 B rows) with one dword direct-to-LDS load,
    // and every lane reads the words of its fragment rows after the barrier.
    // The lane's byte for sub-step s is byte 2s + l/32 of its row's word; the
    // word is shifted by 8 (l/32) so that op_sel 2s picks it.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool sc_a = wv < 4;
    const int sc_row = (sc_a ? row0 : col0) + 64 * (wv & 3) + lane;
    const bool sc_ok = sc_row < (sc_a ? g.M : nb);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(sc_a ? g.sA : g.sB, sc_a ? g.sA_bytes : g.sB_bytes);
    // step-blocked scales: the words of one step's rows are contiguous, so a
    // wave's 64 rows are one 256-byte run
    const uint32_t sc_base = (uint32_t)sc_row * 4u, sc_step = (uint32_t)(sc_a ? g.M : nb) * 4u;
    lds_char* const sc_lds = lsm + KC::LDS_BYTES + (sc_a ? 0 : BM * 4) + 64 * 4 * (wv & 3);
    auto issue_scales = [&](int step) {
      dma4(srs, (sc_ok && step < nk) ? sc_base + sc_step * (uint32_t)step : OOB, sc_lds + (step % NSTAGE) * SC_STAGE);
    };
    const int l32 = lane & 31, sh = 8 * (lane >> 5);
    auto read_scales = [&](int step, uint32_t (&sa)[FM], uint32_t (&sb)[FN]) {
      const char* base = smem + KC::LDS_BYTES + (step % NSTAGE) * SC_STAGE;
#pragma unroll
      for (int i = 0; i < FM; ++i) sa[i] = *(const uint32_t*)(base + (wm * TM + 32 * i + l32) * 4) >> sh;
#pragma unroll
      for (int j = 0; j < FN; ++j) sb[j] = *(const uint32_t*)(base + BM * 4 + (wn * TN + 32 * j + l32) * 4) >> sh;
    };
    FragReaderMX<KC> fra, frb;
    fra.init(wm * TM, lane);
    frb.init(wn * TN, lane);
    i32x8 fa[2][FM], fb[2][FN];
    uint32_t sa[FM], sb[FN], san[FM], sbn[FN];
    auto read_frags = [&](const char* stage, int s, i32x8 (&a)[FM], i32x8 (&b)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = fra.read(stage, s, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = frb.read(stage + OPER_BYTES, s, j);
    };
    // B is the MFMA's first operand (C^T is accumulated), so its scale goes first
#define CODA_MX_MFMAS(S, A_, B_, I0, I1)                                                           \
    _Pragma("unroll") for (int i = (I0); i < (I1); ++i)                                            \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                                 \
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B_[j], A_[i], acc[i][j], 0, 0,   \
                                                                  2 * (S), sb[j], 2 * (S), sa[i]);
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st) {
      issue(st);
      issue_scales(st);
    }
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    __syncthreads();
    read_frags(smem, 0, fa[0], fb[0]);
    read_scales(0, sa, sb);
#if CODA_MX_EARLY_ISSUE
    // the loads of step kt + 2 go out right after step kt's barrier (their
    // stage, step kt's, has been read by then), a step and a quarter before
    // they are waited for; step 1's go out here
    static_assert(NSTAGE == 2, "early issue assumes a two-stage ring");
    issue(1);
    issue_scales(1);
#endif
    for (int kt = 0; kt < nk; ++kt) {
      const char* sc = smem + (kt % NSTAGE) * STAGE_BYTES;
      const char* sn = smem + ((kt + 1) % NSTAGE) * STAGE_BYTES;
#if !CODA_MX_EARLY_ISSUE
      issue(kt + NSTAGE - 1);
      issue_scales(kt + NSTAGE - 1);
#endif
      read_frags(sc, 1, fa[1], fb[1]);
      CODA_MX_MFMAS(0, fa[0], fb[0], 0, FM)
      __builtin_amdgcn_sched_barrier(0);
      // the wait and barrier three quarters through the step (after half of
      // the second sub-step's MFMAs): the next stage's loads get one and a
      // half sub-steps to land, and its first fragments and scales are read
      // under the second half
      CODA_MX_MFMAS(1, fa[1], fb[1], 0, FM / 2)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_NEXT);   // this wave's loads of step kt+1 have landed
      __syncthreads();
#if CODA_MX_EARLY_ISSUE
      issue(kt + 2);
      issue_scales(kt + 2);
#endif
      read_frags(sn, 0, fa[0], fb[0]);
      read_scales(kt + 1, san, sbn);
      CODA_MX_MFMAS(1, fa[1], fb[1], FM / 2, FM)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i) sa[i] = san[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) sb[j] = sbn[j];
    }
#undef CODA_MX_MFMAS
  } else {
  // Software pipeline over a ring of NSTAGE LDS stages (one K step = NSUB
  // MFMA sub-steps of 32 k with 16x16 blocks, of 16 k with 32x32 blocks):
  //   - the direct-to-LDS loads of step k+NSTAGE-1 are issued at the start of
  //     step k into the stage step k-1 used (free since the barrier that ended
  //     step k-1);
  //   - each sub-step issues the MFMAs of its fragments while the fragments
  //     of the next sub-step are read;
  //   - before the last sub-step's MFMAs: wait until this wave's loads of
  //     step k+1 have landed, barrier (all waves' loads of step k+1 are then
  //     in LDS, and every wave is done reading step k-1's stage), and read
  //     step k+1's first fragments while the last MFMAs of step k run.
  // Fragments are double-buffered in registers.  Loads past K read zeros.
  FragReader<AK, KC, BFM, MB> fra;
  FragReader<BKM, KC, BFN, MB> frb;
  fra.init(wm * TM, lane);
  frb.init(wn * TN, lane);
  bf16x8 fa[2][BFM], fb[2][BFN];
  constexpr int NSUB = BK / (MB == 32 ? 16 : 32);

  auto read_frags = [&](const char* stage, int s, bf16x8 (&a)[BFM], bf16x8 (&b)[BFN]) {
#pragma unroll
    for (int i = 0; i < BFM; ++i) a[i] = fra.read(stage, s, i);
#pragma unroll
    for (int j = 0; j < BFN; ++j) b[j] = frb.read(stage + OPER_BYTES, s, j);
  };
  // the MFMAs of block rows [i0, i1)
  auto mfmas_rows = [&](const bf16x8 (&a)[BFM], const bf16x8 (&b)[BFN], int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < BFN; ++j) {
        if constexpr (MB == 16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
      }
  };
  auto mfmas = [&](const bf16x8 (&a)[BFM], const bf16x8 (&b)[BFN]) { mfmas_rows(a, b, 0, BFM); };

  // The compiler interleaves each sub-step's LDS reads and MFMAs; with two
  // waves per SIMD that measured faster than any forced order (all reads
  // first, reads after one MFMA, one read per MFMA).  The four-stage ring
  // issues a stage's loads at the start of the step (right after the
  // barrier, or after the first MFMAs of the last sub-step, measured
  // slower); the two-stage ring issues them right after the barrier (EARLY
  // below).  sched_barrier keeps the sub-steps apart.
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st) issue(st);
  __builtin_amdgcn_s_waitcnt(WAIT_NEXT);     // step 0 has landed
  __syncthreads();
  read_frags(smem, 0, fa[0], fb[0]);
  // measured: faster on every 64-k two-stage loop with four loading waves
  // (the LLaMA-7B dX GEMM 226 -> 218 us already with eight; the first GEMM
  // 234 -> 229 us at the LLaMA-7B shape and 82 -> 80 us at the 1B one)
  constexpr bool EARLY = CODA_BF16_EARLY_ISSUE && NSUB == 2 && NSTAGE == 2;
  if constexpr (EARLY) issue(1);
  if constexpr (NSUB == 2) {
    // Two sub-steps: the wait and barrier go three quarters through the step
    // (after the first half of the last sub-step's MFMAs), so the next
    // stage's loads have as long to land as with four sub-steps, and the
    // next stage's first fragments are read under the second half.  EARLY:
    // the loads of step kt + 2 go out right after step kt's barrier (their
    // stage, step kt's, has been read by then), a step and a quarter before
    // they are waited for.
    for (int kt = 0; kt < nk; ++kt) {
      const char* sc = smem + (kt % NSTAGE) * STAGE_BYTES;
      const char* sn = smem + ((kt + 1) % NSTAGE) * STAGE_BYTES;
      if constexpr (!EARLY) issue(kt + NSTAGE - 1);
      read_frags(sc, 1, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
      __builtin_amdgcn_sched_barrier(0);
      mfmas_rows(fa[1], fb[1], 0, BFM / 2);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_NEXT);   // this wave's loads of step kt+1 have landed
      __syncthreads();
      if constexpr (EARLY) issue(kt + 2);
      read_frags(sn, 0, fa[0], fb[0]);
      mfmas_rows(fa[1], fb[1], BFM / 2, BFM);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (NSUB % 2 == 0) {
    for (int kt = 0; kt < nk; ++kt) {
      const char* sc = smem + (kt % NSTAGE) * STAGE_BYTES;
      const char* sn = smem + ((kt + 1) % NSTAGE) * STAGE_BYTES;
      issue(kt + NSTAGE - 1);
#pragma unroll
      for (int s = 0; s + 1 < NSUB; ++s) {
        read_frags(sc, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
        mfmas(fa[s & 1], fb[s & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(WAIT_NEXT);   // this wave's loads of step kt+1 have landed
      __syncthreads();
      read_frags(sn, 0, fa[0], fb[0]);
      mfmas(fa[(NSUB - 1) & 1], fb[(NSUB - 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // one sub-step per K step: the fragment buffers alternate between steps
    static_assert(NSUB == 1, "odd sub-step counts other than 1");
    auto step1 = [&](int kt, auto bufc) {
      constexpr int b = decltype(bufc)::value;
      issue(kt + NSTAGE - 1);
      __builtin_amdgcn_s_waitcnt(WAIT_NEXT);   // this wave's loads of step kt+1 have landed
      __syncthreads();
      read_frags(smem + ((kt + 1) % NSTAGE) * STAGE_BYTES, 0, fa[b ^ 1], fb[b ^ 1]);
      mfmas(fa[b], fb[b]);
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step1(kt, std::integral_constant<int, 0>{});
      step1(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < nk) step1(kt, std::integral_constant<int, 0>{});
  }
  }
  __builtin_amdgcn_s_waitcnt(0);             // no load may still write into LDS

  // ------------------------------ epilogue ------------------------------
  // The epilogue works on "virtual waves" 64 columns wide: a wave whose tile
  // is TN = 64 NH columns wide runs it NH times, once per 64-column half, so
  // the row-major assignment, the LDS staging and the cross-wave reductions
  // below have the same shape for every wave grid (WM x WNV virtual waves of
  // TM x 64).  Per half, the accumulators are moved, 32 rows (one block row
  // i) at a time, through a wave-private LDS region (32 rows x 64 fp32,
  // 16-byte chunks swizzled by row) into a row-major assignment: in pass p,
  // lane l owns row 32i + 8p + l/8 of the wave tile and its 8 consecutive
  // columns 8(l%8)..+7 of the half.  Every global load and store of the
  // epilogue is then a 16-byte vector and 8 lanes cover one 128-byte row
  // segment.  Only the cross-wave reductions need a workgroup barrier.
  constexpr int VW = 64;                            // virtual wave width
  constexpr int NH = TN / VW;                       // halves per wave
  constexpr int WNV = WNv * NH;                     // virtual waves across the tile
  constexpr int BFNV = VW / MB;                     // MFMA block columns per half
  static_assert(TN % VW == 0 && NH >= 1, "wave tiles are whole 64-column halves");
  const int l32 = lane & 31;
  __syncthreads();                                  // main loop done: LDS is free
  char* region = smem + wave * 8192;
  float* red = (float*)(smem + 8 * 8192);           // [WNV][BM] row partials
  float* redc = red + WNV * BM;                     // [WM][BN] column partials
  const int c8 = lane & 7, rsub = lane >> 3;
  auto dump = [&](int i, int hv) {   // rows 32i..32i+31 of half hv into the region
    if constexpr (MB == 16) {
      // 16x16 blocks (2i, 2i+1): lane l holds row l%16 and columns
      // 16j + 4(l/16)..+3 of block (2i+h, j)
      const int r16 = lane & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < BFNV; ++j) {
          const int row = 16 * h + r16, c = 4 * j + (lane >> 4);
          *(f32x4*)(region + row * 256 + ((c ^ (row & 15)) << 4)) = acc[2 * i + h][hv * BFNV + j];
        }
    } else {
#pragma unroll
      for (int j = 0; j < BFNV; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = j * 8 + 2 * q + (lane >> 5);
          *(f32x4*)(region + l32 * 256 + ((c ^ (l32 & 15)) << 4)) = quad(acc[i][hv * BFNV + j], q);
        }
    }
  };
  auto fetch8 = [&](int r, int cpair, f32x4& lo, f32x4& hi) {   // 8 fp32: columns 8*cpair..+7 of region row r
    lo = *(const f32x4*)(region + r * 256 + (((2 * cpair) ^ (r & 15)) << 4));
    hi = *(const f32x4*)(region + r * 256 + (((2 * cpair + 1) ^ (r & 15)) << 4));
  };
  auto ld8 = [&](const __bf16* p, f32x4& lo, f32x4& hi) {
    const bf16x8 v = *(const bf16x8*)p;
    lo = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    hi = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
  };
  auto st8 = [&](__bf16* p, f32x4 lo, f32x4 hi) {
    *(bf16x8*)p = bf16x8{f2bf(lo[0]), f2bf(lo[1]), f2bf(lo[2]), f2bf(lo[3]),
                         f2bf(hi[0]), f2bf(hi[1]), f2bf(hi[2]), f2bf(hi[3])};
  };
  // EPI_RSQRT_*: r for the tile's rows from the first GEMM's partial sums,
  // summed in the same order as the stand-alone reduction kernel, into rrow
  float* rrow = red + WNV * BM + WMv * BN;          // [BM] row scales
  float* cered = rrow + BM;                         // [WNV][BM] sum-exp partials (EPI_CE_STATS)
  auto tile_row_rsqrt = [&]() {
    if (t < BM) {
      const int row = row0 + t;
      float r = 0.0f;
      if (row < g.M) {
        const float* P = g.part_row + (int64_t)row * g.ld_part_row;
        float sp = 0.0f;
        for (int k = 0; k < g.nparts; ++k) sp += P[k];
        r = 1.0f / sqrtf(sp * g.inv_d + g.eps);
        if (tn == 0) g.r_out[row] = r;
      }
      rrow[t] = r;
    }
    __syncthreads();
  };
  auto sum8 = [](float v) {                          // over the 8 lanes of a row
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    return v;
  };

  if constexpr (EPI == EPI_STORE || EPI == EPI_ROWSCALE || EPI == EPI_RESID_SUMSQ ||
                EPI == EPI_DN || EPI == EPI_SWIGLU_BWD || EPI == EPI_RSQRT_SCALE ||
                EPI == EPI_CE_STATS || EPI == EPI_ROPE) {
    __bf16* C = (__bf16*)g.C;
    if constexpr (EPI == EPI_RSQRT_SCALE) tile_row_rsqrt();
#pragma unroll
    for (int hv = 0; hv < NH; ++hv) {
    const int wnv = wn * NH + hv;                   // virtual wave column
    const int gcol = col0 + wnv * VW + 8 * c8;      // first global column of the lane
    const bool colok = gcol < g.N;
    f32x4 glo{}, ghi{}, clo{0.f, 0.f, 0.f, 0.f}, chi{0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI == EPI_DN || EPI == EPI_RESID_SUMSQ) {
      if (colok && g.vcol) ld8((const __bf16*)g.vcol + gcol, glo, ghi);
    }
    // The passes' global inputs (E's 8 columns of the row, the row's scale,
    // its label) are loaded one row group ahead, so that their latency hides
    // under the previous group's passes instead of stalling every pass.
    constexpr bool PRE_E = EPI == EPI_RESID_SUMSQ || EPI == EPI_DN || EPI == EPI_SWIGLU_BWD;
    bf16x8 epre[2][4], upre[2][4];
    float vpre[2][4];
    int lpre[2][4];
    auto prefetch = [&](int i, int b) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = row0 + wm * TM + i * 32 + 8 * p + rsub;
        const bool ok = colok && row < g.M;
        const __bf16* ep = (const __bf16*)g.E + (int64_t)row * g.lde + gcol;
        if constexpr (PRE_E) epre[b][p] = ok ? *(const bf16x8*)ep : bf16x8{};
        if constexpr (EPI == EPI_SWIGLU_BWD) upre[b][p] = ok ? *(const bf16x8*)(ep + g.F) : bf16x8{};
        if constexpr (EPI == EPI_ROWSCALE)
          vpre[b][p] = ok ? (g.vrow ? g.vrow[row] : bf2f(((const __bf16*)g.vcol)[row])) : 0.0f;
        if constexpr (EPI == EPI_DN) vpre[b][p] = ok ? g.vrow[row] : 0.0f;
        if constexpr (EPI == EPI_CE_STATS) lpre[b][p] = ok ? g.labels[row] : -1;
      }
    };
    auto unpack8 = [](const bf16x8& v, f32x4& lo, f32x4& hi) {
      lo = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
      hi = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
    };
    prefetch(0, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i + 1 < FM) prefetch(i + 1, (i + 1) & 1);
      wave_lds_sync();                              // the previous pass's reads are done
      dump(i, hv);
      __builtin_amdgcn_s_waitcnt(0xc07f);           // this wave's LDS writes are done
      wave_lds_sync();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = 8 * p + rsub;
        const int lrow_t = wm * TM + i * 32 + r;     // row within the workgroup tile
        const int row = row0 + lrow_t;
        const bool ok = colok && row < g.M;
        f32x4 lo, hi;
        fetch8(r, c8, lo, hi);
        const int64_t o = (int64_t)row * g.ldc + gcol;
        if constexpr (EPI == EPI_STORE) {
          if (ok) st8(C + o, lo, hi);
        } else if constexpr (EPI == EPI_ROPE) {
          // the lane's 8 columns are 4 pairs of one head (the head width is a
          // multiple of 8); cos and sin of their angles from the table
          if (ok) {
            if (gcol < g.rope_rot) {
              const int hd = g.rope_head >> 1;
              const int64_t ti = (int64_t)(row % g.rope_seq) * hd + ((gcol % g.rope_head) >> 1);
              const f32x4 cs = *(const f32x4*)(g.rope_tab + ti);
              const f32x4 sn = *(const f32x4*)(g.rope_tab + (int64_t)g.rope_seq * hd + ti);
              f32x4 rlo, rhi;
              rlo[0] = lo[0] * cs[0] - lo[1] * sn[0];
              rlo[1] = lo[0] * sn[0] + lo[1] * cs[0];
              rlo[2] = lo[2] * cs[1] - lo[3] * sn[1];
              rlo[3] = lo[2] * sn[1] + lo[3] * cs[1];
              rhi[0] = hi[0] * cs[2] - hi[1] * sn[2];
              rhi[1] = hi[0] * sn[2] + hi[1] * cs[2];
              rhi[2] = hi[2] * cs[3] - hi[3] * sn[3];
              rhi[3] = hi[2] * sn[3] + hi[3] * cs[3];
              st8(C + o, rlo, rhi);
            } else {
              st8(C + o, lo, hi);
            }
          }
        } else if constexpr (EPI == EPI_ROWSCALE) {
          if (ok) {
            const float sc = vpre[i & 1][p];
            st8(C + o, lo * sc, hi * sc);
          }
        } else if constexpr (EPI == EPI_RSQRT_SCALE) {
          if (ok) {
            const float sc = rrow[lrow_t];
            st8(C + o, lo * sc, hi * sc);
          }
        } else if constexpr (EPI == EPI_RESID_SUMSQ) {
          float s = 0.0f;
          if (ok) {
            f32x4 elo, ehi;
            unpack8(epre[i & 1][p], elo, ehi);
            lo += elo;
            hi += ehi;
            st8(C + o, lo, hi);
            if constexpr (FMT == FMT_MX8) {
            } else if (g.C2) {
              if (g.c2_trans) {                         // y * gamma back into the region
                *(f32x4*)(region + r * 256 + (((2 * c8) ^ (r & 15)) << 4)) = lo * glo;
                *(f32x4*)(region + r * 256 + (((2 * c8 + 1) ^ (r & 15)) << 4)) = hi * ghi;
              } else {
                st8((__bf16*)g.C2 + (int64_t)row * g.ldc2 + gcol, lo * glo, hi * ghi);
              }
            }
            const f32x4 sq = lo * lo + hi * hi;
            s = sq[0] + sq[1] + sq[2] + sq[3];
          }
          s = sum8(s);
          if (c8 == 0) red[wnv * BM + lrow_t] = s;
          if constexpr (FMT == FMT_MX8) {
            // y * gamma to MXFP8: the 4 lanes c8 = 4b..4b+3 hold one 32-column
            // block of the row; shared exponent floor(log2 amax) - 8 (clamped
            // at -127) from amax's exponent field, elements scaled by the
            // exact power of two, saturated at 448 and rounded to nearest
            // even by the hardware conversion
            f32x4 vlo = lo * glo, vhi = hi * ghi;
            float am = 0.0f;
            if (ok) {
#pragma unroll
              for (int e = 0; e < 4; ++e) am = fmaxf(am, fmaxf(fabsf(vlo[e]), fabsf(vhi[e])));
            }
            am = fmaxf(am, __shfl_xor(am, 1));
            am = fmaxf(am, __shfl_xor(am, 2));
            const int sexp = max((int)((__float_as_uint(am) >> 23) & 255) - 135, -127);
            const float inv = __uint_as_float((uint32_t)(127 - sexp) << 23);
            auto sat = [&](float v) { return mx8_sat(v, inv); };
            int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(vlo[0]), sat(vlo[1]), 0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(vlo[2]), sat(vlo[3]), w0, true);
            int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(vhi[0]), sat(vhi[1]), 0, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat(vhi[2]), sat(vhi[3]), w1, true);
            if (ok) {
              *(uint2*)(g.q_out + (int64_t)row * g.ldq + gcol) = uint2{(uint32_t)w0, (uint32_t)w1};
              if ((c8 & 3) == 0)   // step-blocked: [d/128][M][4]
                g.qs_out[((int64_t)(gcol >> 7) * g.M + row) * 4 + ((gcol >> 5) & 3)] = (uint8_t)(sexp + 127);
            }
          }
        } else if constexpr (EPI == EPI_DN) {
          // dh = acc; dn = gamma dh (stored); row sum of dn*y; column sums of dh*r*y
          float s = 0.0f;
          if (ok) {
            f32x4 ylo, yhi;
            unpack8(epre[i & 1][p], ylo, yhi);
            const float rv = vpre[i & 1][p];
            const f32x4 dlo = lo * glo, dhi = hi * ghi;
            st8(C + o, dlo, dhi);
            if (g.C2) st8((__bf16*)g.C2 + (int64_t)row * g.ldc2 + gcol, ylo * rv, yhi * rv);
            const f32x4 sp = dlo * ylo + dhi * yhi;
            s = sp[0] + sp[1] + sp[2] + sp[3];
            clo += lo * ylo * rv;
            chi += hi * yhi * rv;
          }
          s = sum8(s);
          if (c8 == 0) red[wnv * BM + lrow_t] = s;
        } else if constexpr (EPI == EPI_CE_STATS) {
          // logits stored; the stateful max / sum-exp of the row over this
          // half's 64 columns (8 lanes x 8), columns past N left out
          float mx = -INFINITY;
          if (ok) {
            st8(C + o, lo, hi);
            mx = fmaxf(fmaxf(fmaxf(lo[0], lo[1]), fmaxf(lo[2], lo[3])),
                       fmaxf(fmaxf(hi[0], hi[1]), fmaxf(hi[2], hi[3])));
            const int lab = lpre[i & 1][p];
            if (lab >= gcol && lab < gcol + 8) {
              const int e = lab - gcol;
              g.lab_out[row] = e < 4 ? lo[e] : hi[e - 4];
            }
          }
          mx = fmaxf(mx, __shfl_xor(mx, 1));
          mx = fmaxf(mx, __shfl_xor(mx, 2));
          mx = fmaxf(mx, __shfl_xor(mx, 4));
          float se = 0.0f;
          if (ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) se += __expf(lo[e] - mx) + __expf(hi[e] - mx);
          }
          se = sum8(se);
          if (c8 == 0) {
            red[wnv * BM + lrow_t] = mx;
            cered[wnv * BM + lrow_t] = se;
          }
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          // da = acc [M, F]; g, u from the saved gu; dgu = [dg | du]
          f32x4 dg0{0.f, 0.f, 0.f, 0.f}, dg1 = dg0, du0 = dg0, du1 = dg0;   // zero out of range
          if (ok) {
            f32x4 g0, g1, u0, u1;
            unpack8(epre[i & 1][p], g0, g1);
            unpack8(upre[i & 1][p], u0, u1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float sg = sigmoid_f(g0[e]);
              dg0[e] = lo[e] * u0[e] * sg * (1.0f + g0[e] * (1.0f - sg));
              du0[e] = lo[e] * g0[e] * sg;
              sg = sigmoid_f(g1[e]);
              dg1[e] = hi[e] * u1[e] * sg * (1.0f + g1[e] * (1.0f - sg));
              du1[e] = hi[e] * g1[e] * sg;
            }
            if (C) {
              st8(C + o, dg0, dg1);
              st8(C + o + g.F, du0, du1);
            }
          }
          if constexpr (FMT == FMT_MX8) {
            // dgu as stored (bf16) to MXFP8 without storing it: along 2F here
            // (the 4 lanes c8 = 4b..4b+3 of a row hold a 32-column block of
            // dg, and of du; step-blocked scales [2F/128][M][4]), and along M
            // after the group's passes, from the bf16 values kept in this
            // row of the region (whose fp32 accumulators this pass has read)
            f32x4 b0, b1, c0, c1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              b0[e] = bf2f(f2bf(dg0[e]));
              b1[e] = bf2f(f2bf(dg1[e]));
              c0[e] = bf2f(f2bf(du0[e]));
              c1[e] = bf2f(f2bf(du1[e]));
            }
            if (g.q_out) {
              int sg_, su_;
              const uint2 wg = mx8_block_of_4_lanes(b0, b1, sg_);
              const uint2 wu = mx8_block_of_4_lanes(c0, c1, su_);
              if (ok) {
                *(uint2*)(g.q_out + (int64_t)row * g.ldq + gcol) = wg;
                *(uint2*)(g.q_out + (int64_t)row * g.ldq + g.F + gcol) = wu;
                if ((c8 & 3) == 0) {
                  const int cu = g.F + gcol;
                  g.qs_out[((int64_t)(gcol >> 7) * g.M + row) * 4 + ((gcol >> 5) & 3)] = (uint8_t)(sg_ + 127);
                  g.qs_out[((int64_t)(cu >> 7) * g.M + row) * 4 + ((cu >> 5) & 3)] = (uint8_t)(su_ + 127);
                }
              }
            }
            if (g.qt_out) {
              wave_lds_sync();                      // after this pass's region reads
              *(bf16x8*)(region + r * 256 + c8 * 16) =
                  bf16x8{f2bf(b0[0]), f2bf(b0[1]), f2bf(b0[2]), f2bf(b0[3]),
                         f2bf(b1[0]), f2bf(b1[1]), f2bf(b1[2]), f2bf(b1[3])};
              *(bf16x8*)(region + r * 256 + 128 + c8 * 16) =
                  bf16x8{f2bf(c0[0]), f2bf(c0[1]), f2bf(c0[2]), f2bf(c0[3]),
                         f2bf(c1[0]), f2bf(c1[1]), f2bf(c1[2]), f2bf(c1[3])};
            }
          }
        }
      }
      if constexpr (EPI == EPI_SWIGLU_BWD && FMT == FMT_MX8) {
        // dgu along M: the region holds the group's 32 rows x [dg 64 | du 64]
        // (bf16); lane l quantises column l of dg and of du over those rows
        // (the transposing quantiser's arithmetic) into codes [2F][ldqt] and
        // scales [M/128][2F][4]
        if (g.qt_out) {
          __builtin_amdgcn_s_waitcnt(0xc07f);         // this wave's LDS writes are done
          wave_lds_sync();
          const int rowT = row0 + wm * TM + i * 32;
          const int colT = col0 + wnv * VW + lane;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float v[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) v[e] = bf2f(*(const __bf16*)(region + e * 256 + h2 * 128 + lane * 2));
            uint32_t w[8];
            const int sexp = mx8_block32(v, w);
            if (colT < g.N && rowT < g.M) {
              const int64_t cT = (int64_t)colT + h2 * g.F;
              uint8_t* dst = g.qt_out + cT * g.ldqt + rowT;
              *(uint4*)dst = uint4{w[0], w[1], w[2], w[3]};
              *(uint4*)(dst + 16) = uint4{w[4], w[5], w[6], w[7]};
              g.qts_out[((int64_t)(rowT >> 7) * (2 * g.F) + cT) * 4 + ((rowT >> 5) & 3)] = (uint8_t)(sexp + 127);
            }
          }
        }
      }
      if constexpr (EPI == EPI_RESID_SUMSQ) {
        // y * gamma transposed: C2[col][row].  In pass q, lanes 4c..4c+3 take
        // column 16q + c of the half's 64 and rows 8(l%4)..+7 each, so one
        // store instruction writes 16 columns x 64 contiguous bytes.
        if (FMT == FMT_BF16 && g.C2 && g.c2_trans) {
          __builtin_amdgcn_s_waitcnt(0xc07f);         // this wave's LDS writes are done
          wave_lds_sync();
          const int rg = 8 * (lane & 3);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = 16 * q + (lane >> 2);
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = rg + e;
              v[e] = *(const float*)(region + r * 256 + (((c >> 2) ^ (r & 15)) << 4) + (c & 3) * 4);
            }
            const int colT = col0 + wnv * VW + c;
            const int rowT = row0 + wm * TM + i * 32 + rg;
            if (colT < g.N && rowT < g.M)
              *(bf16x8*)((__bf16*)g.C2 + (int64_t)colT * g.ldc2 + rowT) =
                  bf16x8{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3]),
                         f2bf(v[4]), f2bf(v[5]), f2bf(v[6]), f2bf(v[7])};
          }
        }
      }
    }
    if constexpr (EPI == EPI_DN) {
      // column partials of this half: reduce over the 8 row groups of lanes
      // (l/8); the WM waves that share these columns combine through LDS below
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        clo[e] += __shfl_xor(clo[e], 8);
        clo[e] += __shfl_xor(clo[e], 16);
        clo[e] += __shfl_xor(clo[e], 32);
        chi[e] += __shfl_xor(chi[e], 8);
        chi[e] += __shfl_xor(chi[e], 16);
        chi[e] += __shfl_xor(chi[e], 32);
      }
      if (lane < 8) {
        *(f32x4*)(redc + wm * BN + wnv * VW + 8 * c8) = clo;
        *(f32x4*)(redc + wm * BN + wnv * VW + 8 * c8 + 4) = chi;
      }
    }
    }   // halves
    if constexpr (EPI == EPI_CE_STATS) {
      // combine the WNV virtual waves' (max, sum-exp) of each row in order; a
      // virtual wave whose columns all lie past N left (max -inf, sum 0) and
      // is skipped by its zero sum; a NaN logit made its sum NaN, which the
      // row keeps (fmaxf alone would drop it)
      __syncthreads();
      if (t < BM) {
        const int row = row0 + t;
        float m = red[t];
        for (int w = 1; w < WNV; ++w) m = fmaxf(m, red[w * BM + t]);
        float sm = 0.0f;
        for (int w = 0; w < WNV; ++w) {
          const float sw = cered[w * BM + t];
          if (sw != 0.0f) sm += sw * __expf(red[w * BM + t] - m);
        }
        if (row < g.M) {
          g.part_row[(int64_t)row * g.ld_part_row + tn] = m;
          g.part_col[(int64_t)row * g.ld_part_row + tn] = sm;
        }
      }
    }
    if constexpr (EPI == EPI_RESID_SUMSQ || EPI == EPI_DN) {
      __syncthreads();
      if (t < BM) {
        const int row = row0 + t;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WNV; ++w) s += red[w * BM + t];
        if (row < g.M) g.part_row[(int64_t)row * g.ld_part_row + tn] = s;
      }
      if constexpr (EPI == EPI_DN) {
        if (t < BN) {
          const int col = col0 + t;
          float s = 0.0f;
#pragma unroll
          for (int w = 0; w < WMv; ++w) s += redc[w * BN + t];
          if (col < g.N) g.part_col[(int64_t)tm * g.ld_part_col + col] = s;
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_RSQRT_SWIGLU) {
    // Each half's 64 columns are 32 gate columns j and the 32 up columns of
    // the same j.  Pass p: lane l owns row 16p + l/4 and gate/up column group
    // l%4 (8 columns each).  EPI_RSQRT_SWIGLU first scales both by the row's
    // RMS factor r (the GEMM's A operand is the un-normalised y gamma).
    if constexpr (EPI == EPI_RSQRT_SWIGLU) tile_row_rsqrt();
    __bf16* GU = (__bf16*)g.C;
    __bf16* Aout = (__bf16*)g.C2;
    const int c4 = lane & 3, r4 = lane >> 2;
#pragma unroll
    for (int hv = 0; hv < NH; ++hv) {
    const int jj = tn * (BN / 2) + (wn * NH + hv) * (VW / 2) + 8 * c4;
    const bool jok = jj < g.F;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      wave_lds_sync();                              // the previous pass's reads are done
      dump(i, hv);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      wave_lds_sync();
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int r = 16 * p + r4;
        const int row = row0 + wm * TM + i * 32 + r;
        f32x4 g0, g1, u0, u1;
        fetch8(r, c4, g0, g1);
        fetch8(r, 4 + c4, u0, u1);
        if constexpr (EPI == EPI_RSQRT_SWIGLU) {
          const float sc = rrow[wm * TM + i * 32 + r];
          g0 *= sc;
          g1 *= sc;
          u0 *= sc;
          u1 *= sc;
        }
        f32x4 a0, a1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0[e] = silu_f(g0[e]) * u0[e];
          a1[e] = silu_f(g1[e]) * u1[e];
        }
        const bool ok = jok && row < g.M;
        if (ok) {
          st8(GU + (int64_t)row * g.ldc + jj, g0, g1);
          st8(GU + (int64_t)row * g.ldc + g.F + jj, u0, u1);
          st8(Aout + (int64_t)row * g.ldc2 + jj, a0, a1);
        }
        if constexpr (FMT == FMT_MX8) {
          // a (as stored, bf16) to MXFP8 along F for the down GEMM: the 4
          // lanes c4 = 0..3 of a row hold its 32-block jj0..jj0+31
          // (jj0 = jj - 8 c4, a multiple of 32); step-blocked scales
          // [F/128][M][4]
          f32x4 b0 = f32x4{0.f, 0.f, 0.f, 0.f}, b1 = b0;
          if (ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              b0[e] = bf2f(f2bf(a0[e]));
              b1[e] = bf2f(f2bf(a1[e]));
            }
          }
          int sexp;
          const uint2 w = mx8_block_of_4_lanes(b0, b1, sexp);
          if (ok) {
            *(uint2*)(g.q_out + (int64_t)row * g.ldq + jj) = w;
            if (c4 == 0) g.qs_out[((int64_t)(jj >> 7) * g.M + row) * 4 + ((jj >> 5) & 3)] = (uint8_t)(sexp + 127);
          }
        }
      }
    }
    }   // halves
  }
}

// WIN: operands reached through windows (an operand past 2 GiB); else one
// buffer descriptor per operand (the plain, slightly faster loaders).
template <int WMv, int WNv, int BKv, int NSTv, bool AK, bool BKM, int EPI, bool WIN>
__global__ void __launch_bounds__(64 * WMv * WNv)
    __attribute__((amdgpu_waves_per_eu(WMv * WNv / 4, WMv * WNv / 4)))
gemm_bf16_kernel(GemmArgs g) {
  gemm_body<FMT_BF16, WMv, WNv, BKv, NSTv, AK, BKM, EPI, WIN>(g);
}

template <int WMv, int WNv, int EPI, bool WIN>
__global__ void __launch_bounds__(64 * WMv * WNv)
    __attribute__((amdgpu_waves_per_eu(WMv * WNv / 4, WMv * WNv / 4)))
gemm_mx8_kernel(GemmArgs g) {
  gemm_body<FMT_MX8, WMv, WNv, 64, 2, true, true, EPI, WIN>(g);
}

// bf16 rows -> MXFP8 along the row.  A lane takes 8 consecutive elements
// (one 16-byte load), 4 lanes one 32-block: shared exponent and element
// rounding as in the first GEMM's epilogue; scales stored step-blocked
// ([cols/128][rows][4]).  A workgroup takes G x 256 groups of 8 of one row
// (blockIdx.x: the chunk of the row, blockIdx.y: the first row, strided by
// gridDim.y); a thread issues its G loads before it quantises any, so that
// they are in flight together.  Every lane takes part in the shuffles
// (cols % 32 == 0 keeps a 32-block's 4 lanes together and either all in
// range or all out).
template <int G>
__global__ void __launch_bounds__(256) mx8_quantize_kernel(const __bf16* __restrict__ src, int64_t ld,
                                                           int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int gpr = (int)(cols / 8);                  // groups of 8 per row
  const int g0 = (int)blockIdx.x * (256 * G) + (int)threadIdx.x;
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
    const __bf16* s_row = src + row * ld;
    bf16x8 v[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int g = g0 + 256 * k;
      v[k] = g < gpr ? *(const bf16x8*)(s_row + (int64_t)g * 8) : bf16x8{};
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int g = g0 + 256 * k;
      const f32x4 lo{(float)v[k][0], (float)v[k][1], (float)v[k][2], (float)v[k][3]};
      const f32x4 hi{(float)v[k][4], (float)v[k][5], (float)v[k][6], (float)v[k][7]};
      int sexp;
      const uint2 w = mx8_block_of_4_lanes(lo, hi, sexp);
      if (g < gpr) {
        const int64_t col = (int64_t)g * 8;
        *(uint2*)(codes + row * cols + col) = w;
        if ((g & 3) == 0) scales[((col >> 7) * rows + row) * 4 + ((col >> 5) & 3)] = (uint8_t)(sexp + 127);
      }
    }
  }
}

// Column position of element (r, c) in the 128 x 64 staging tile of the
// column quantisers: 16-byte piece c / 8 of row r moves to piece
// (c / 8) ^ 2 (r / 32 % 4), so that the four 32-row blocks a group of 4
// lanes reads (one column, blocks b = 0..3) fall in different banks.
__device__ __forceinline__ int qt_col(int r, int c) { return ((((c >> 3) ^ (((r >> 5) & 3) << 1))) << 3) | (c & 7); }

// bf16 [rows, cols] -> MXFP8 along the columns' direction, stored transposed:
// codes [cols][rows] (a column's 32-blocks of consecutive rows are contiguous
// 32 bytes), scales step-blocked [rows/128][cols][4].  This is the operand
// layout of a GEMM that contracts over the rows (X^T dy, n^T dz).  A
// workgroup stages a 128 x 64 tile in LDS (each 16-byte row piece read
// once); thread t = 4c + b then quantises column c's rows 32b..32b+31
// exactly as the row quantiser does a 32-block and writes its 32 codes as
// two 16-byte stores, so that the 4 lanes of a column fill one 128-byte run
// of the output.  rows % 128 == 0.
__global__ void __launch_bounds__(256) mx8_quantize_t_kernel(const __bf16* __restrict__ src, int64_t ld,
                                                             int64_t rows, int64_t cols,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  __shared__ __bf16 tile[128][64];
  // one-dimensional grid, column blocks fastest: block (rb, cb)
  const uint32_t ncb = (uint32_t)((cols + 63) / 64);
  const uint32_t rb = blockIdx.x / ncb, cb = blockIdx.x - rb * ncb;
  const int64_t row0 = (int64_t)rb * 128, col0 = (int64_t)cb * 64;
  const int t = threadIdx.x;
  // 1024 pieces of 8 values, 4 per thread.  A piece past the last column
  // reads the row's last piece instead (cols % 8 == 0) and stages zeros, so
  // the four loads carry no branch and are in flight together.
  bf16x8 raw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int piece = t + 256 * k;
    const int r = piece >> 3, c8 = (piece & 7) * 8;
    raw[k] = *(const bf16x8*)(src + (row0 + r) * ld + min(col0 + c8, cols - 8));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int piece = t + 256 * k;
    const int r = piece >> 3, c8 = (piece & 7) * 8;
    *(bf16x8*)&tile[r][qt_col(r, c8)] = col0 + c8 < cols ? raw[k] : bf16x8{};
  }
  __syncthreads();
  const int c = t >> 2, b = t & 3;        // column, 32-row block
  const int64_t col = col0 + c;
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = (float)tile[32 * b + e][qt_col(32 * b, c)];
  uint32_t w[8];
  const int sexp = mx8_block32(v, w);
  if (col < cols) {
    uint8_t* dst = codes + col * rows + row0 + 32 * b;
    *(uint4*)dst = uint4{w[0], w[1], w[2], w[3]};
    *(uint4*)(dst + 16) = uint4{w[4], w[5], w[6], w[7]};
    scales[((int64_t)rb * cols + col) * 4 + b] = (uint8_t)(sexp + 127);
  }
}

// The MXFP8 operands of the block's backward that come from one bf16 [rows,
// cols] tensor, in one pass over it (rows % 128 == 0):
//   QUANT_SRC: v = src; quantised along the row (codes qr [rows][cols], scales
//              sr [cols/128][rows][4]; cols % 128 == 0) and along the column,
//              stored transposed (codes qt [cols][rows], scales st
//              [rows/128][cols][4]) -- dz for the dh and dW2 GEMMs;
//   QUANT_DY:  v = dy = r_i dn - c_i y (+ dy_in when given; bf16), written
//              over dn (src = out = dR); quantised both ways -- dy for the
//              dX and dW1 GEMMs;
//   QUANT_NROW: v = n = r_i y (bf16; src = y); quantised along the column
//              only -- n for the dW2 GEMM.
// With qr NULL only the transposed codes are made; with gated_F > 0 (a
// gate/up weight [d, 2F], F % 32 == 0) they are written in gate/up order.
// The values are rounded to bf16 before they are quantised (the stored dn,
// n and dy of the bf16 backward).  A workgroup takes a 128 x 64 tile: each
// thread produces 4 pieces of 8 values, quantises them along the row with
// its 3 neighbours (the row quantiser's arithmetic), and stages them in LDS;
// thread 4c + b then quantises column c's rows 32b..32b+31 as the transposed
// quantiser does.
enum QuantMode : int { QUANT_SRC = 0, QUANT_DY = 1, QUANT_NROW = 2 };
template <int MODE>
__global__ void __launch_bounds__(256) mx8_quantize_fused_kernel(MxQuantArgs q) {
  __shared__ __bf16 tile[128][64];
  // one-dimensional grid, column blocks fastest: block (rb, cb)
  const uint32_t ncb = (uint32_t)((q.cols + 63) / 64);
  const uint32_t rb = blockIdx.x / ncb, cb = blockIdx.x - rb * ncb;
  const int64_t row0 = (int64_t)rb * 128, col0 = (int64_t)cb * 64;
  const int t = threadIdx.x;
  // 1024 pieces of 8 values, 4 per thread.  Every operand of the 4 pieces is
  // loaded before any is used, a piece past the last column reading the
  // row's last piece (cols % 8 == 0; its values are dropped), so the loads
  // carry no branch and are in flight together.
  bf16x8 a[4], yv[4], din[4];
  float ri[4], ci[4];
  const bool has_din = MODE == QUANT_DY && q.dy_in;   // uniform over the grid
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int piece = t + 256 * k;
    const int64_t row = row0 + (piece >> 3), col = min(col0 + (piece & 7) * 8, q.cols - 8);
    a[k] = *(const bf16x8*)((const __bf16*)q.src + row * q.ld + col);
    if constexpr (MODE == QUANT_DY) {
      yv[k] = *(const bf16x8*)((const __bf16*)q.y + row * q.ld + col);
      ci[k] = q.c[row];
      if (has_din) din[k] = *(const bf16x8*)((const __bf16*)q.dy_in + row * q.ld + col);
    }
    if constexpr (MODE != QUANT_SRC) ri[k] = q.r[row];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int piece = t + 256 * k;
    const int r = piece >> 3, c8 = (piece & 7) * 8;
    const int64_t row = row0 + r, col = col0 + c8;
    const bool ok = col < q.cols;
    bf16x8 v{};
    if constexpr (MODE == QUANT_SRC) {
      v = a[k];
    } else if constexpr (MODE == QUANT_DY) {
      if (has_din) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f2bf(ri[k] * bf2f(a[k][e]) - ci[k] * bf2f(yv[k][e]) + bf2f(din[k][e]));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f2bf(ri[k] * bf2f(a[k][e]) - ci[k] * bf2f(yv[k][e]));
      }
      if (ok) *(bf16x8*)((__bf16*)q.out + row * q.ld + col) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = f2bf(ri[k] * bf2f(a[k][e]));
    }
    if (!ok) v = bf16x8{};
    *(bf16x8*)&tile[r][qt_col(r, c8)] = v;
    if (MODE != QUANT_NROW && q.qr) {             // uniform over the grid
      const f32x4 lo{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
      const f32x4 hi{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
      int sexp;
      const uint2 w = mx8_block_of_4_lanes(lo, hi, sexp);
      if (ok) {
        *(uint2*)(q.qr + row * q.cols + col) = w;
        if ((col & 31) == 0) q.sr[((col >> 7) * q.rows + row) * 4 + ((col >> 5) & 3)] = (uint8_t)(sexp + 127);
      }
    }
  }
  __syncthreads();
  const int c = t >> 2, b = t & 3;        // column, 32-row block (4 lanes per column)
  const int64_t col = col0 + c;
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = (float)tile[32 * b + e][qt_col(32 * b, c)];
  uint32_t w[8];
  const int sexp = mx8_block32(v, w);
  if (col < q.cols) {
    // gated_F: column c of a [.., 2F] gate/up weight goes to row 64 (j / 32)
    // + 32 [c is an up column] + j % 32, j = c mod F (the order of a gated
    // tile's columns)
    int64_t tr = col;
    if (q.gated_F > 0) {
      const int64_t j = col < q.gated_F ? col : col - q.gated_F;
      tr = 64 * (j >> 5) + (col < q.gated_F ? 0 : 32) + (j & 31);
    }
    uint8_t* dst = q.qt + tr * q.rows + row0 + 32 * b;
    *(uint4*)dst = uint4{w[0], w[1], w[2], w[3]};
    *(uint4*)(dst + 16) = uint4{w[4], w[5], w[6], w[7]};
    q.st[((int64_t)rb * q.cols + tr) * 4 + b] = (uint8_t)(sexp + 127);
  }
}

// ---------------------------------------------------------------------------
// fp32 forward path: an LDS-tiled GEMM on the fp32 matrix instruction
// (v_mfma_f32_16x16x4f32) with the same epilogue semantics.  A is [M,K] (k
// contiguous), B is [K,N].  A 64x64 tile, four waves of 32x32 (2x2 blocks of
// 16x16), K staged 16 at a time.  In a 16x16x4 block lane l supplies
// A[l%16][l/16] and B[l/16][l%16] and holds C[4(l/16)+q][l%16], q = 0..3.
// The accumulators go through LDS to a 4x4-per-thread layout for the
// epilogue.
// ---------------------------------------------------------------------------
constexpr int FT = kTileF32;
constexpr int FK = 16;

template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g) {
  __shared__ float sA[FK][FT + 4];
  __shared__ float sB[FK][FT + 4];
  __shared__ float sC[FT][FT + 1];
  __shared__ float red[FT][17];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lk = lane >> 4;
  const int tiles_n = (g.N + FT - 1) / FT;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int row0 = tm * FT, col0 = tn * FT;
  const float* A = (const float*)g.A;
  const float* B = (const float*)g.B;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < g.K; k0 += FK) {
    for (int e = t; e < FT * FK; e += 256) {
      const int m = e / FK, k = e % FK;
      const int gr = row0 + m, gk = k0 + k;
      sA[k][m] = (gr < g.M && gk < g.K) ? A[(int64_t)gr * g.lda + gk] : 0.0f;
      const int kk = e / FT, n = e % FT;
      const int gk2 = k0 + kk, gc = col0 + n;
      sB[kk][n] = (gk2 < g.K && gc < g.N) ? B[(int64_t)gk2 * g.ldb + gc] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; k += 4) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sA[k + lk][wm * 32 + 16 * i + l16];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = sB[k + lk][wn * 32 + 16 * j + l16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sC[wm * 32 + 16 * i + 4 * lk + q][wn * 32 + 16 * j + l16] = acc[i][j][q];
  __syncthreads();
  float* C = (float*)g.C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + ty * 4 + i;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = col0 + tx * 4 + j;
      if (row < g.M && col < g.N) {
        float v = sC[ty * 4 + i][tx * 4 + j];
        if constexpr (EPI == EPI_RESID_SUMSQ) {
          v += ((const float*)g.E)[(int64_t)row * g.lde + col];
          s += v * v;
          if (g.C2) ((float*)g.C2)[(int64_t)row * g.ldc2 + col] = v * ((const float*)g.vcol)[col];
        } else if constexpr (EPI == EPI_ROWSCALE) {
          v *= g.vrow[row];
        }
        C[(int64_t)row * g.ldc + col] = v;
      }
    }
    if constexpr (EPI == EPI_RESID_SUMSQ) red[ty * 4 + i][tx] = s;
  }
  if constexpr (EPI == EPI_RESID_SUMSQ) {
    __syncthreads();
    if (t < FT) {
      const int row = row0 + t;
      float s = 0.0f;
      for (int x = 0; x < 16; ++x) s += red[t][x];
      if (row < g.M) g.part_row[(int64_t)row * g.ld_part_row + tn] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------
__global__ void row_rsqrt_kernel(const float* __restrict__ P, int64_t ldp, int T, int64_t M,
                                 float inv_d, float eps, float* __restrict__ r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M) return;
  float s = 0.0f;
  for (int k = 0; k < T; ++k) s += P[i * ldp + k];
  r[i] = 1.0f / sqrtf(s * inv_d + eps);
}

// c and dgamma.  Rows: four lanes per row, each summing every fourth partial
// (consecutive lanes read consecutive 16-byte pieces of the [M][Tn] array),
// then two shuffles.  Columns: one lane per column over the Tm row tiles.
// Every sum has a fixed order, so the result is run-to-run identical.
__global__ void bwd_reduce_kernel(const float* __restrict__ S, int64_t lds, int Tn,
                                  const float* __restrict__ r, int64_t M, float inv_d,
                                  const float* __restrict__ G, int Tm, int64_t d,
                                  float* __restrict__ c, float* __restrict__ dgamma) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row_threads = ((M * 4 + 255) / 256) * 256;   // whole blocks for the row part
  if (v < row_threads) {
    const int64_t i = v >> 2;
    const int q = (int)(v & 3);
    float s = 0.0f;
    if (i < M) {
#pragma unroll 4
      for (int k = q; k < Tn; k += 4) s += S[i * lds + k];
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (i < M && q == 0) {
      const float ri = r[i];
      c[i] = ri * ri * ri * s * inv_d;
    }
  } else {
    const int64_t j = v - row_threads;
    if (j >= d) return;
    float s = 0.0f;
#pragma unroll 8
    for (int k = 0; k < Tm; ++k) s += G[(int64_t)k * d + j];
    dgamma[j] = s;
  }
}

__global__ void dy_kernel(__bf16* __restrict__ dR, const __bf16* __restrict__ y,
                          const float* __restrict__ r, const float* __restrict__ c,
                          const __bf16* __restrict__ dy_in, int64_t M, int64_t d) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = v * 8;
  if (e0 >= M * d) return;
  const int64_t i = e0 / d;
  const float ri = r[i], ci = c[i];
  const bf16x8 dn = *(const bf16x8*)(dR + e0);
  const bf16x8 yv = *(const bf16x8*)(y + e0);
  bf16x8 o;
  if (dy_in) {
    const bf16x8 din = *(const bf16x8*)(dy_in + e0);
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = f2bf(ri * bf2f(dn[k]) - ci * bf2f(yv[k]) + bf2f(din[k]));
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = f2bf(ri * bf2f(dn[k]) - ci * bf2f(yv[k]));
  }
  *(bf16x8*)(dR + e0) = o;
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Wave grid of every bf16 and MXFP8 GEMM: 2 x 4 waves of 128 x 64 (two per
// SIMD).  A 2 x 2 grid of 128 x 128 wave tiles (one wave per SIMD, a third
// fewer LDS reads per MFMA) measured 13-15% slower: with no second wave on the
// SIMD its stalls are not covered, and it still ran into the power limit.
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kMxWavesM = kWavesM, kMxWavesN = kWavesN;

// K step / ring depth: 64 x 2 when an operand is K-contiguous, else 32 x 4.
// A GEMM with a K-contiguous A and an N-contiguous B operand (the forward
// layout) whose operands together take more than half the MALL (the 256 MiB
// memory-side cache) also takes 32 x 4 (DEEP): much of its loads then see
// HBM latency, which loads two 32-k steps ahead hide better than three
// quarters of a 64-k step, and that outweighs the shorter 64-byte rows
// (measured, 32 x 4 against 64 x 2: the SwiGLU gate/up GEMM 9% faster, the
// down GEMM 5%, the LM-head logits GEMM 4%, the rotary QKV GEMM 2.5%, the
// 70B-hidden first GEMM 1.3%).  With both operands K-contiguous the 64 x 2
// ring, whose loads go out a step and a quarter ahead from one wave per
// SIMD, is faster at every size measured (the dh GEMM of the RMSNorm
// backward 4.5% at the LLaMA-7B shape and 9% at the 70B-hidden shape, the
// SwiGLU dX GEMM 10% and da GEMM 8%, the LM-head dh GEMM 8%, the rotary dX
// GEMM 10%, the 70B-hidden dX GEMM 5%).
#ifndef CODA_DEEP_MIN_MIB
#define CODA_DEEP_MIN_MIB 128
#endif
constexpr int64_t kDeepMinBytes = (int64_t)CODA_DEEP_MIN_MIB << 20;

// an operand that one 32-bit buffer descriptor cannot cover
static bool needs_windows(const GemmArgs& g) { return g.A_total > kMaxWindow || g.B_total > kMaxWindow; }

template <bool AK, bool BKM, int EPI, bool DEEP = false>
static hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  static_assert(!DEEP || (AK && !BKM), "the deep ring is for the forward layout (A K-, B N-contiguous)");
  constexpr int BKv = (AK || BKM) && !DEEP ? 64 : 32;
  constexpr int NSTv = (AK || BKM) && !DEEP ? 2 : 4;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (EPI == EPI_SWIGLU || EPI == EPI_RSQRT_SWIGLU) ? (g.N + BN / 2 - 1) / (BN / 2)
                                                                      : (g.N + BN - 1) / BN;
  if (needs_windows(g))
    hipLaunchKernelGGL((gemm_bf16_kernel<kWavesM, kWavesN, BKv, NSTv, AK, BKM, EPI, true>),
                       dim3(tiles_m * tiles_n), dim3(64 * kWavesM * kWavesN), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<kWavesM, kWavesN, BKv, NSTv, AK, BKM, EPI, false>),
                       dim3(tiles_m * tiles_n), dim3(64 * kWavesM * kWavesN), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& g, bool ak, bool bk, Epi epi, hipStream_t s) {
  // The combinations the block uses:
  //   forward GEMMs:      A k-major, B mn-major  (X W1, X W, a Wd)
  //   input gradients:    A k-major, B k-major   (dz W2^T, dy W1^T, dz Wd^T, dgu W^T)
  //   both mn-major:      (y gamma)^T-stored times W2, and the weight
  //                       gradients n^T dz, X^T dy, a^T dz, X^T dgu
  if (ak && !bk) {
    const bool deep = ((int64_t)g.M + g.N) * g.K * 2 > kDeepMinBytes;
    switch (epi) {
      case EPI_STORE:
        return deep ? launch_one<true, false, EPI_STORE, true>(g, s) : launch_one<true, false, EPI_STORE>(g, s);
      case EPI_RESID_SUMSQ:
        return deep ? launch_one<true, false, EPI_RESID_SUMSQ, true>(g, s)
                    : launch_one<true, false, EPI_RESID_SUMSQ>(g, s);
      case EPI_CE_STATS:
        return deep ? launch_one<true, false, EPI_CE_STATS, true>(g, s)
                    : launch_one<true, false, EPI_CE_STATS>(g, s);
      case EPI_ROPE:
        return deep ? launch_one<true, false, EPI_ROPE, true>(g, s) : launch_one<true, false, EPI_ROPE>(g, s);
      case EPI_RSQRT_SCALE:
        return deep ? launch_one<true, false, EPI_RSQRT_SCALE, true>(g, s)
                    : launch_one<true, false, EPI_RSQRT_SCALE>(g, s);
      case EPI_SWIGLU:
        return deep ? launch_one<true, false, EPI_SWIGLU, true>(g, s) : launch_one<true, false, EPI_SWIGLU>(g, s);
      default: break;
    }
  } else if (ak && bk) {
    switch (epi) {
      case EPI_STORE: return launch_one<true, true, EPI_STORE>(g, s);
      case EPI_DN: return launch_one<true, true, EPI_DN>(g, s);
      case EPI_SWIGLU_BWD: return launch_one<true, true, EPI_SWIGLU_BWD>(g, s);
      default: break;
    }
  } else if (!ak && !bk) {
    switch (epi) {
      case EPI_STORE: return launch_one<false, false, EPI_STORE>(g, s);
      case EPI_ROWSCALE: return launch_one<false, false, EPI_ROWSCALE>(g, s);
      case EPI_RSQRT_SCALE: return launch_one<false, false, EPI_RSQRT_SCALE>(g, s);
      case EPI_RSQRT_SWIGLU: return launch_one<false, false, EPI_RSQRT_SWIGLU>(g, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <int EPI>
static hipError_t launch_mx8_one(const GemmArgs& g, hipStream_t s) {
  constexpr bool gated = EPI == EPI_SWIGLU || EPI == EPI_RSQRT_SWIGLU;
  const int tiles = ((g.M + BM - 1) / BM) * (gated ? (g.N + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN);
  if (needs_windows(g))
    hipLaunchKernelGGL((gemm_mx8_kernel<kMxWavesM, kMxWavesN, EPI, true>), dim3(tiles),
                       dim3(64 * kMxWavesM * kMxWavesN), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_mx8_kernel<kMxWavesM, kMxWavesN, EPI, false>), dim3(tiles),
                       dim3(64 * kMxWavesM * kMxWavesN), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_mx8(const GemmArgs& g, Epi epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_mx8_one<EPI_STORE>(g, s);
    case EPI_RESID_SUMSQ: return launch_mx8_one<EPI_RESID_SUMSQ>(g, s);
    case EPI_RSQRT_SCALE: return launch_mx8_one<EPI_RSQRT_SCALE>(g, s);
    case EPI_DN: return launch_mx8_one<EPI_DN>(g, s);
    case EPI_ROWSCALE: return launch_mx8_one<EPI_ROWSCALE>(g, s);
    case EPI_SWIGLU: return launch_mx8_one<EPI_SWIGLU>(g, s);
    case EPI_RSQRT_SWIGLU: return launch_mx8_one<EPI_RSQRT_SWIGLU>(g, s);
    case EPI_SWIGLU_BWD: return launch_mx8_one<EPI_SWIGLU_BWD>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mx8_quantize_t(const void* src, int64_t ld, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  // (cols / 64 rounded up) x (rows / 128) blocks in one dimension: rows up
  // to 2^23 would overflow the 65535 limit of a second grid dimension
  const int64_t blocks = (cols + 63) / 64 * (rows / 128);
  if (blocks < 1 || blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL(mx8_quantize_t_kernel, grid, dim3(256), 0, s, (const __bf16*)src, ld, rows, cols, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_mx8_quantize_fused(const MxQuantArgs& q, int mode, hipStream_t s) {
  const int64_t blocks = (q.cols + 63) / 64 * (q.rows / 128);   // as the transposing quantiser
  if (blocks < 1 || blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  switch (mode) {
    case QUANT_SRC: hipLaunchKernelGGL(mx8_quantize_fused_kernel<QUANT_SRC>, grid, dim3(256), 0, s, q); break;
    case QUANT_DY: hipLaunchKernelGGL(mx8_quantize_fused_kernel<QUANT_DY>, grid, dim3(256), 0, s, q); break;
    case QUANT_NROW: hipLaunchKernelGGL(mx8_quantize_fused_kernel<QUANT_NROW>, grid, dim3(256), 0, s, q); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx8_quantize(const void* src, int64_t ld, int64_t rows, int64_t cols,
                               uint8_t* codes, uint8_t* scales, hipStream_t s) {
  // groups of 8 per thread (1, 2 or 4): the count that leaves the fewest
  // threads of a row's last chunk idle, the larger on a tie; rows beyond the
  // grid's 65535 are strided
  const int64_t gpr = cols / 8;
  int G = 4;
  int64_t idle = (gpr + 1023) / 1024 * 1024 - gpr;
  for (int g : {2, 1}) {
    const int64_t per = 256 * (int64_t)g, i = (gpr + per - 1) / per * per - gpr;
    if (i < idle) {
      idle = i;
      G = g;
    }
  }
  const dim3 grid((unsigned)((gpr + 256 * G - 1) / (256 * G)), (unsigned)std::min<int64_t>(rows, 65535));
  if (G == 4)
    hipLaunchKernelGGL(mx8_quantize_kernel<4>, grid, dim3(256), 0, s, (const __bf16*)src, ld, rows, cols, codes,
                       scales);
  else if (G == 2)
    hipLaunchKernelGGL(mx8_quantize_kernel<2>, grid, dim3(256), 0, s, (const __bf16*)src, ld, rows, cols, codes,
                       scales);
  else
    hipLaunchKernelGGL(mx8_quantize_kernel<1>, grid, dim3(256), 0, s, (const __bf16*)src, ld, rows, cols, codes,
                       scales);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& g, Epi epi, hipStream_t s) {
  const int tiles = ((g.M + FT - 1) / FT) * ((g.N + FT - 1) / FT);
  switch (epi) {
    case EPI_RESID_SUMSQ:
      hipLaunchKernelGGL((gemm_f32_kernel<EPI_RESID_SUMSQ>), dim3(tiles), dim3(256), 0, s, g);
      break;
    case EPI_ROWSCALE:
      hipLaunchKernelGGL((gemm_f32_kernel<EPI_ROWSCALE>), dim3(tiles), dim3(256), 0, s, g);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL((gemm_f32_kernel<EPI_STORE>), dim3(tiles), dim3(256), 0, s, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_row_rsqrt(const float* P, int64_t ldp, int T, int64_t M, int64_t d, float eps,
                            float* r, hipStream_t s) {
  hipLaunchKernelGGL(row_rsqrt_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, P, ldp,
                     T, M, 1.0f / (float)d, eps, r);
  return hipGetLastError();
}

__global__ void rope_table_kernel(float* __restrict__ tab, int S, int D, double base) {
  const int hd = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)S * hd) return;
  const int p = (int)(idx / hd), i = (int)(idx % hd);
  const double ang = (double)p * pow(base, -2.0 * (double)i / (double)D);
  tab[idx] = (float)cos(ang);
  tab[(int64_t)S * hd + idx] = (float)sin(ang);
}

__global__ void rope_inverse_kernel(const __bf16* __restrict__ dY, const float* __restrict__ tab,
                                    __bf16* __restrict__ dP, int64_t M, int64_t N, int N_rot, int D,
                                    int S) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = v * 8;
  if (e0 >= M * N) return;
  const int64_t m = e0 / N;
  const int64_t c0 = e0 - m * N;
  const bf16x8 x = *(const bf16x8*)(dY + e0);
  if (c0 >= N_rot) {
    *(bf16x8*)(dP + e0) = x;
    return;
  }
  const int hd = D >> 1;
  const int64_t ti = (int64_t)(m % S) * hd + ((c0 % D) >> 1);
  const f32x4 cs = *(const f32x4*)(tab + ti);
  const f32x4 sn = *(const f32x4*)(tab + (int64_t)S * hd + ti);
  bf16x8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = bf2f(x[2 * k]), b = bf2f(x[2 * k + 1]);
    o[2 * k] = f2bf(a * cs[k] + b * sn[k]);
    o[2 * k + 1] = f2bf(-a * sn[k] + b * cs[k]);
  }
  *(bf16x8*)(dP + e0) = o;
}

hipError_t launch_rope_table(float* tab, int S, int D, double base, hipStream_t s) {
  const int64_t n = (int64_t)S * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tab, S, D,
                     base);
  return hipGetLastError();
}

hipError_t launch_rope_inverse(const void* dY, const float* tab, void* dP, int64_t M, int64_t N,
                               int N_rot, int D, int S, hipStream_t s) {
  const int64_t chunks = (M * N) / 8;
  hipLaunchKernelGGL(rope_inverse_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     (const __bf16*)dY, tab, (__bf16*)dP, M, N, N_rot, D, S);
  return hipGetLastError();
}

// One wave per row: lane l folds the row's tiles l, l + 64, ... into a running
// (max, sum-exp) pair, then the 64 lanes combine in a fixed butterfly order.
// A pair is rescaled only when its sum is non-zero: an empty pair (-inf, 0)
// adds nothing, and a NaN sum (a NaN logit in that tile) stays NaN.  A row
// whose label lies outside [0, V) is ignored: loss 0 (its lse is still formed).
__device__ __forceinline__ float ce_rescale(float s, float m, float nm) {
  return s != 0.0f ? s * __expf(m - nm) : 0.0f;
}
__global__ void ce_combine_kernel(const float* __restrict__ pmax, const float* __restrict__ psum,
                                  int64_t ldp, int T, const float* __restrict__ lab,
                                  const int* __restrict__ labels, int64_t V, int64_t M,
                                  float* __restrict__ lse, float* __restrict__ loss) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float m = -INFINITY, sm = 0.0f;
  if (row < M) {
    for (int t = lane; t < T; t += 64) {
      const float mt = pmax[row * ldp + t], st = psum[row * ldp + t];
      const float nm = fmaxf(m, mt);
      sm = ce_rescale(sm, m, nm) + ce_rescale(st, mt, nm);
      m = nm;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o), so = __shfl_xor(sm, o);
    const float nm = fmaxf(m, mo);
    sm = ce_rescale(sm, m, nm) + ce_rescale(so, mo, nm);
    m = nm;
  }
  if (row < M && lane == 0) {
    const float l = m + __logf(sm);
    const int lb = labels[row];
    lse[row] = l;
    loss[row] = (lb >= 0 && lb < V) ? l - lab[row] : 0.0f;
  }
}

__global__ void ce_dlogits_kernel(const __bf16* __restrict__ logits, const int* __restrict__ labels,
                                  const float* __restrict__ lse, const float* __restrict__ dloss,
                                  __bf16* __restrict__ dlogits, int64_t M, int64_t V) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = v * 8;
  if (e0 >= M * V) return;
  const int64_t i = e0 / V;
  const int64_t j0 = e0 - i * V;
  const float li = lse[i];
  const int lab = labels[i];
  const float di = (lab >= 0 && lab < V) ? dloss[i] : 0.0f;   // an ignored row has no gradient
  const bf16x8 x = *(const bf16x8*)(logits + e0);
  bf16x8 o;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float pk = __expf(bf2f(x[k]) - li);
    o[k] = f2bf(di * (pk - (j0 + k == lab ? 1.0f : 0.0f)));
  }
  *(bf16x8*)(dlogits + e0) = o;
}

hipError_t launch_ce_combine(const float* pmax, const float* psum, int64_t ldp, int T,
                             const float* lab, const int* labels, int64_t V, int64_t M, float* lse,
                             float* loss, hipStream_t s) {
  hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, pmax, psum,
                     ldp, T, lab, labels, V, M, lse, loss);
  return hipGetLastError();
}

hipError_t launch_ce_dlogits(const void* logits, const int* labels, const float* lse,
                             const float* dloss, void* dlogits, int64_t M, int64_t V, hipStream_t s) {
  const int64_t chunks = (M * V) / 8;
  hipLaunchKernelGGL(ce_dlogits_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     (const __bf16*)logits, labels, lse, dloss, (__bf16*)dlogits, M, V);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const float* S, int64_t lds, int Tn, const float* r, int64_t M,
                             int64_t d, const float* G, int Tm, float* c, float* dgamma,
                             hipStream_t s) {
  const int64_t threads = ((M * 4 + 255) / 256) * 256 + d;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, S,
                     lds, Tn, r, M, 1.0f / (float)d, G, Tm, d, c, dgamma);
  return hipGetLastError();
}

hipError_t launch_dy(void* dR, const void* y, const float* r, const float* c, const void* dy_in,
                     int64_t M, int64_t d, hipStream_t s) {
  const int64_t chunks = (M * d) / 8;
  hipLaunchKernelGGL(dy_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     (__bf16*)dR, (const __bf16*)y, r, c, (const __bf16*)dy_in, M, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Built-in scratch for callers that cannot allocate device memory
// (coda_fwd_noalloc): a file-scope device array, one copy per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device copy, so its device address is looked up
// once per device (with that device current) and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mtx;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mtx);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace coda
