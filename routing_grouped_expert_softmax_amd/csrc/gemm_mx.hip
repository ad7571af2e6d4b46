// gemm_mx.hip — device-scheduled grouped GEMM on MXFP8 operands (E4M3 codes
// with one e8m0 scale per 32 elements along K) for the SwiGLU experts, on the
// gfx950 scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), fp32
// accumulation, bf16 outputs.  MXFP8 for the expert FFN follows the first
// page, section 三 (MXFP8 for selected operations; the gain comes from the
// FFN and expert data movement).
//
// Every operand arrives K-contiguous from the quantiser (weights are
// quantised along their GEMM's K and stored transposed where needed), so one
// tile layout serves all modes: 8-row groups of 1 KiB, [16-byte chunk][row %
// 8][16 bytes], the chunk index XOR-ed with bit 3 of the row (conflict-free 16
// lane passes).  A tile row holds 128 K values (4 scale blocks); its four
// scale bytes arrive with it as one 32-bit LDS word per row.
//
// Operand layout of the scaled MFMA (checked on the device): lane l supplies
// row (l & 31), and its bytes 0-15 / 16-31 hold K = 16*(l>>5) + 0..15 and
// 32 + 16*(l>>5) + 0..15 of the 64-wide step; the scale of K block 0 comes
// from the lanes with l < 32, of block 1 from the lanes with l >= 32.  So a
// lane reads chunks (4kk + half) and (4kk + 2 + half) and scale byte
// (2kk + half) of its row.
//
// Scheduling, stages and the epilogue are the bf16 kernel's (gemm_common.h).
// Tiles are 256 x 256 x 128 in two stages, one block per CU, eight waves
// (64 x 128 wave tiles, 128 accumulator registers, two waves per SIMD, one
// scale-row load per wave): 6-15 % faster per mode than four waves of
// 128 x 128 (one wave per SIMD, nothing to hide the LDS and barrier latency).
// The register budget of 256 per wave holds with the code-load offsets kept
// as two per-lane values plus uniform row steps.
// Wgrad operands are the column-quantised per-expert token blocks: expert e's
// K range starts at the exclusive scan of roundup(n_e, 128).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "gemm_common.h"
#include "mx.h"

using namespace moe;
using namespace moe_gemm;

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

struct MxParams {
  const uint8_t* a0;   // A codes (segment 0)
  const uint8_t* a1;   // A codes, second K segment (gate/up dgrad)
  const uint8_t* sa0;  // A scales
  const uint8_t* sa1;
  int lda;              // bytes per A row
  const uint8_t* b0;   // B codes (or first of the pair / first K segment)
  const uint8_t* b1;
  const uint8_t* sb0;
  const uint8_t* sb1;
  int ldb;              // bytes per B row
  long long b_row_e;    // per-expert row offset of B (row-quantised weights)
  long long b_k_e;      // per-expert K offset of B (column-quantised weights)
  void* c0;
  void* c1;
  void* c2;
  int ldc;
  long long c_gstride;
  const bf16_t* aux0;
  const bf16_t* aux1;
  const int32_t* offsets;
  int E;
  int M;
  int N;
  int K;
  int kseg;
  int ntiles;
  int mtiles;
  const int32_t* kbase;  // K-ragged: padded K start of each expert (exclusive scan of roundup(n_e, 128))
};

constexpr int BK = 128;  // K bytes (= fp8 values) per stage

// Tile of NW waves in an (NW/2) x 2 grid: each wave a (BM/(NW/2)) x 128
// sub-tile.  Code rows move in 1 KiB loads (8 rows), scale rows in 256-byte
// loads (64 rows).  When the scale loads of A and B add up to NW, wave w
// issues exactly one: A's for the first waves, B's for the rest.
template <int BM, int NW = 4>
struct MxTile {
  static constexpr int WM = BM / (NW / 2);
  static constexpr int SM = WM / 32;
  static constexpr int A_BYTES = BM * BK;
  static constexpr int B_BYTES = BN * BK;
  static constexpr int AS_BYTES = BM * 4;  // one 32-bit scale word per row
  static constexpr int BS_BYTES = BN * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES;
  static constexpr int A_INST = A_BYTES / 1024 / NW;  // 16-byte loads per wave
  static constexpr int B_INST = B_BYTES / 1024 / NW;
  static constexpr int AS_TOT = AS_BYTES / 256, BS_TOT = BS_BYTES / 256;
  static constexpr bool SPLIT = NW > 4 && AS_TOT + BS_TOT == NW;
  static constexpr int AS_INST = SPLIT ? 0 : AS_TOT / NW;  // 4-byte loads per wave
  static constexpr int BS_INST = SPLIT ? 0 : BS_TOT / NW;
  static constexpr int S_INST = SPLIT ? 1 : AS_INST + BS_INST;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "code loads per wave");
  static_assert(SPLIT || (AS_TOT % NW == 0 && BS_TOT % NW == 0), "scale loads per wave");
};

template <int MODE, int BM, int S, int NW>
__global__ void __launch_bounds__(64 * NW, 1) grouped_gemm_mx_kernel(MxParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using TR = Traits<MODE>;
  using TL = MxTile<BM, NW>;
  constexpr int SM = TL::SM;
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds2[S > 2 ? TL::STAGE : 16];
  __shared__ int sh[kThreads + 4];

  const int tid = threadIdx.x;
  const int lane_in = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wv >> 1, wn = wv & 1;

  // ---------------------------------------------------------------- work
  // Row-ragged modes: one tile per block from eight equal-count XCD ranges.
  // K-ragged modes: eight equal-cost XCD ranges (tiles cost as much as their
  // expert's rows); block b takes tiles first + b / 8, + nslot, ... of its
  // XCD's range.
  Work w0;
  int first = 0, end = 1, nslot = 1, L0 = 0;
  if (TR::kKRAGGED) {
    kragged_xcd_range<BK>(p.offsets, p.E, p.ntiles * p.mtiles, blockIdx.x & 7, first, end);
    nslot = gridDim.x >> 3;
    L0 = first + (int)(blockIdx.x >> 3);
  } else {
    if (!find_mtile<BM>(p.E, p.offsets, p.ntiles, sh, w0)) return;
  }
  for (int L = L0; L < end; L += nslot) {
  // Blocks of the K-ragged modes walk several tiles.  The lane id is made
  // opaque at each tile, so the per-lane offsets derived from it are formed
  // again per tile rather than held through the epilogue: held, they pushed
  // these kernels past their 256 registers, and the spill reloads inside
  // the K loop waited for the next stage's loads.
  int lane = lane_in;
  if constexpr (TR::kKRAGGED) asm volatile("" : "+v"(lane));
  Work w = w0;
  int kbase = 0;  // K-ragged: first K byte of the expert in the padded layout
  if (TR::kKRAGGED) {
    // the previous tile's epilogue has finished with the LDS stage buffers
    if (L != L0) lds_barrier();
    // expert-major, then m-tile, then n-tile (n fastest)
    const int per_e = p.ntiles * p.mtiles;
    w.e = L / per_e;
    const int r = L % per_e;
    w.nt = r % p.ntiles;
    w.m0 = (r / p.ntiles) * BM;
    kbase = __builtin_amdgcn_readfirstlane(p.kbase[w.e]);  // padded K start of the expert
    const int n = p.offsets[w.e + 1] - p.offsets[w.e];
    w.row0 = kbase;
    w.rows = (n + 127) / 128 * 128;  // padded K of the expert (padding is zero)
  }
  const int nk = TR::kKRAGGED ? w.rows / BK : p.K / BK;

  // ---------------------------------------------------------------- sources
  rsrc_t ra0, ra1, rsa0, rsa1, rb0, rb1, rsb0, rsb1;
  if (TR::kKRAGGED) {
    // codes [M][lda] and [N][ldb] from K byte kbase on; rows m0.. of A
    ra0 = make_rsrc(p.a0 + kbase, (unsigned long long)p.M * p.lda - kbase);
    rsa0 = make_rsrc(p.sa0 + kbase / 32, (unsigned long long)p.M * (p.lda / 32) - kbase / 32);
    rb0 = make_rsrc(p.b0 + kbase, (unsigned long long)p.N * p.ldb - kbase);
    rsb0 = make_rsrc(p.sb0 + kbase / 32, (unsigned long long)p.N * (p.ldb / 32) - kbase / 32);
    rb1 = TR::kDUAL ? make_rsrc(p.b1 + kbase, (unsigned long long)p.N * p.ldb - kbase) : rb0;
    rsb1 = TR::kDUAL
               ? make_rsrc(p.sb1 + kbase / 32, (unsigned long long)p.N * (p.ldb / 32) - kbase / 32)
               : rsb0;
    ra1 = ra0;
    rsa1 = rsa0;
  } else {
    // A: the tile's rows; B: the expert's weights (row and/or K offset)
    const unsigned long long ab = (unsigned long long)w.rows * p.lda;
    ra0 = make_rsrc(p.a0 + (size_t)w.row0 * p.lda, ab);
    rsa0 = make_rsrc(p.sa0 + (size_t)w.row0 * (p.lda / 32), ab / 32);
    ra1 = ra0;
    rsa1 = rsa0;
    if (MODE == DGRAD_UP) {
      ra1 = make_rsrc(p.a1 + (size_t)w.row0 * p.lda, ab);
      rsa1 = make_rsrc(p.sa1 + (size_t)w.row0 * (p.lda / 32), ab / 32);
    }
    const size_t bo = (size_t)w.e * p.b_row_e * p.ldb + (size_t)w.e * p.b_k_e;
    const unsigned long long bb = (unsigned long long)p.N * p.ldb - (size_t)w.e * p.b_k_e;
    rb0 = make_rsrc(p.b0 + bo, bb);
    rsb0 = make_rsrc(p.sb0 + bo / 32, bb / 32);
    const bool two = TR::kDUAL || MODE == DGRAD_UP;
    rb1 = two ? make_rsrc(p.b1 + bo, bb) : rb0;
    rsb1 = two ? make_rsrc(p.sb1 + bo / 32, bb / 32) : rsb0;
  }

  // Per-lane offsets of this wave's direct loads.  Code tiles: instruction q
  // fills rows 8q..8q+7; lane = physical chunk * 8 + row % 8, and the source
  // chunk is the physical one XOR bit 3 of the row.  Scale tiles: 64 rows per
  // instruction, one 32-bit word (4 scale blocks) per lane.
  const int lda_s = p.lda / 32, ldb_s = p.ldb / 32;
  static_assert(TL::A_INST % 2 == 0 && TL::B_INST % 2 == 0, "code loads come in even/odd pairs");
  // Code loads j and j + 2 of a wave are 16 rows apart with the same swizzle:
  // two per-lane offsets (j even, odd) plus a uniform 16-row step each.
  int aoff[2], boff[2], asoff[TL::AS_INST + 1], bsoff[TL::BS_INST + 1];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = wv * TL::A_INST + j;
    const int row = q * 8 + (lane & 7), c = (lane >> 3) ^ ((row >> 3) & 1);
    aoff[j] = (TR::kKRAGGED ? (w.m0 + row) : row) * p.lda + c * 16;
  }
#pragma unroll
  for (int j = 0; j < TL::AS_INST; ++j) {
    const int row = (wv * TL::AS_INST + j) * 64 + lane;
    asoff[j] = (TR::kKRAGGED ? (w.m0 + row) : row) * lda_s;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = wv * TL::B_INST + j;
    const int row = q * 8 + (lane & 7), c = (lane >> 3) ^ ((row >> 3) & 1);
    // dual: rows 0..127 of the tile from matrix 0, 128..255 from matrix 1
    const int n = TR::kDUAL ? w.nt * 128 + (row & 127) : w.nt * BN + row;
    boff[j] = n * p.ldb + c * 16;
  }
#pragma unroll
  for (int j = 0; j < TL::BS_INST; ++j) {
    const int row = (wv * TL::BS_INST + j) * 64 + lane;
    const int n = TR::kDUAL ? w.nt * 128 + (row & 127) : w.nt * BN + row;
    bsoff[j] = n * ldb_s;
  }
  // One scale load per wave: 64 rows of A (wv < AS_TOT) or of B starting at
  // the uniform row s_row0, lane l taking row s_row0 + l.  Its per-lane
  // offset l * ld is formed at each issue from the lane id: kept across the
  // K loop it was spilled in the K-ragged modes, and its reload before the
  // load waited for every load in flight.
  [[maybe_unused]] const bool s_is_a = wv < TL::AS_TOT;
  [[maybe_unused]] int s_row0 = 0;
  if constexpr (TL::SPLIT) {
    const int sw = s_is_a ? wv : wv - TL::AS_TOT;
    if (s_is_a)
      s_row0 = (TR::kKRAGGED ? w.m0 : 0) + sw * 64;
    else  // dual: rows 0..127 of the tile from matrix 0, 128..255 from matrix 1
      s_row0 = TR::kDUAL ? w.nt * 128 + ((sw * 64) & 127) : w.nt * BN + sw * 64;
  }

  auto stage_ptr = [&](auto st) -> LDS_AS unsigned char* {
    constexpr int ST = decltype(st)::value;
    if constexpr (ST == 0) return (LDS_AS unsigned char*)lds0;
    else if constexpr (ST == 1) return (LDS_AS unsigned char*)lds1;
    else return (LDS_AS unsigned char*)lds2;
  };
  auto issue = [&](int kt, auto st) {
    const int k0 = kt * BK;
    LDS_AS unsigned char* base = stage_ptr(st);
    const bool seg1 = (MODE == DGRAD_UP) && k0 >= p.kseg;
    const int kk = seg1 ? k0 - p.kseg : k0;
    const rsrc_t ra = seg1 ? ra1 : ra0, rsa = seg1 ? rsa1 : rsa0;
    rsrc_t rb = seg1 ? rb1 : rb0, rsb = seg1 ? rsb1 : rsb0;
    // dual: the upper half of the waves fills the second matrix's code rows
    // (and, one scale load per wave each, its scale rows)
    [[maybe_unused]] const rsrc_t rsb_split = (TR::kDUAL && wv - TL::AS_TOT >= 2) ? rsb1 : rsb;
    if (TR::kDUAL && wv >= NW / 2) {
      rb = rb1;
      rsb = rsb1;
    }
#pragma unroll
    for (int j = 0; j < TL::A_INST; ++j)
      dma16(ra, (LDS_AS void*)(base + (wv * TL::A_INST + j) * 1024), aoff[j & 1],
            kk + (j >> 1) * 16 * p.lda);
#pragma unroll
    for (int j = 0; j < TL::B_INST; ++j)
      dma16(rb, (LDS_AS void*)(base + TL::A_BYTES + (wv * TL::B_INST + j) * 1024), boff[j & 1],
            kk + (j >> 1) * 16 * p.ldb);
    // dual scale rows: waves 0,1 rows 0..127 (matrix 0), 2,3 rows 128..255
#pragma unroll
    for (int j = 0; j < TL::AS_INST; ++j)
      dma4(rsa, (LDS_AS void*)(base + TL::A_BYTES + TL::B_BYTES + (wv * TL::AS_INST + j) * 256),
           asoff[j], kk / 32);
#pragma unroll
    for (int j = 0; j < TL::BS_INST; ++j)
      dma4(rsb,
           (LDS_AS void*)(base + TL::A_BYTES + TL::B_BYTES + TL::AS_BYTES +
                          (wv * TL::BS_INST + j) * 256),
           bsoff[j], kk / 32);
    if constexpr (TL::SPLIT) {
      const int ld_s = s_is_a ? lda_s : ldb_s;
      const int lid = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      // rows past the operand fail the buffer range check and read as zero
      const int voff = (s_row0 + lid) * ld_s;
      if (s_is_a)
        dma4(rsa, (LDS_AS void*)(base + TL::A_BYTES + TL::B_BYTES + wv * 256), voff, kk / 32);
      else
        dma4(rsb_split,
             (LDS_AS void*)(base + TL::A_BYTES + TL::B_BYTES + TL::AS_BYTES + (wv - TL::AS_TOT) * 256),
             voff, kk / 32);
    }
  };

  // ---------------------------------------------------------------- fragments
  // Code fragment of 32 rows (row0 + lane & 31) for 64-wide step kk: chunks
  // 4kk + half and 4kk + 2 + half, each XOR-ed with bit 3 of the row.
  const int h = lane >> 5;
  const int cl = ((lane & 31) >> 3) * 1024 + ((h ^ (((lane & 31) >> 3) & 1)) * 128) + (lane & 7) * 16;
  // (two 16-byte vector halves joined by a shuffle, so the reads land in the
  // operand's registers without copies)
  auto frag = [&](const LDS_AS unsigned char* t, int row0, int kk) -> i32x8 {
    const LDS_AS unsigned char* a = t + (row0 >> 3) * 1024 + kk * 512 + cl;
    const i32x4 lo = *(const LDS_AS i32x4*)(a);
    const i32x4 hi = *(const LDS_AS i32x4*)(a + 256);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Scale word of the lane's row, shifted so byte 2kk is block 2kk + half.
  auto sword = [&](const LDS_AS unsigned char* s, int row0) -> int {
    const unsigned v = *(const LDS_AS unsigned*)(s + (row0 + (lane & 31)) * 4);
    return (int)(v >> (8 * h));
  };

  f32x16 acc[SM][4];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](auto st) {
    const LDS_AS unsigned char* As = stage_ptr(st);
    const LDS_AS unsigned char* Bs = As + TL::A_BYTES;
    const LDS_AS unsigned char* Ass = Bs + TL::B_BYTES;
    const LDS_AS unsigned char* Bss = Ass + TL::AS_BYTES;
    int sx[4], sy[SM];
#pragma unroll
    for (int sn = 0; sn < 4; ++sn) {
      const int row0 = TR::kDUAL ? (sn >> 1) * 128 + wn * 64 + (sn & 1) * 32 : wn * 128 + sn * 32;
      sx[sn] = sword(Bss, row0);
    }
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) sy[sm] = sword(Ass, wm * TL::WM + sm * 32);
    // one 64-wide step; the opsel byte index must be a compile-time constant
    auto mstep = [&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      i32x8 xb[4], ya[SM];
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) {
        const int row0 = TR::kDUAL ? (sn >> 1) * 128 + wn * 64 + (sn & 1) * 32 : wn * 128 + sn * 32;
        xb[sn] = frag(Bs, row0, kk);
      }
#pragma unroll
      for (int sm = 0; sm < SM; ++sm) ya[sm] = frag(As, wm * TL::WM + sm * 32, kk);
#pragma unroll
      for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < 4; ++sn)
          acc[sm][sn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              xb[sn], ya[sm], acc[sm][sn], 0, 0, 2 * kk, sx[sn], 2 * kk, sy[sm]);
    };
    mstep(std::integral_constant<int, 0>{});
    mstep(std::integral_constant<int, 1>{});
    // The empty asm takes every accumulator, so all MFMAs of this stage are
    // issued before the next step's wait for its loads.  Without it the
    // compiler moved them below that wait, and the wait had nothing to
    // overlap (one load latency exposed per pair of steps).
#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) asm volatile("" : "+v"(acc[sm][sn]));
  };

  // ---------------------------------------------------------------- main loop
  constexpr int LPS = TL::A_INST + TL::B_INST + TL::S_INST;  // loads per wave per stage
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (0 < nk) issue(0, I0{});
  if (S > 2 && 1 < nk) issue(1, I1{});
  auto step = [&](int kt, auto cur, auto nxt) {
    const int after = min(S - 2, nk - 1 - kt);
    if (S >= 3 && after >= 1)
      __builtin_amdgcn_s_waitcnt((LPS & 15) | (7 << 4) | (15 << 8) | ((LPS >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (kt + S - 1 < nk) issue(kt + S - 1, nxt);
    compute(cur);
  };
  int kt = 0;
  if constexpr (S == 2) {
    for (; kt + 1 < nk; kt += 2) {
      step(kt, I0{}, I1{});
      step(kt + 1, I1{}, I0{});
    }
    if (kt < nk) step(kt, I0{}, I1{});
  } else {
    for (; kt + 2 < nk; kt += 3) {
      step(kt, I0{}, I2{});
      step(kt + 1, I1{}, I0{});
      step(kt + 2, I2{}, I1{});
    }
    if (kt < nk) step(kt, I0{}, I2{});
    if (kt + 1 < nk) step(kt + 1, I1{}, I0{});
  }
  asm volatile("s_barrier" ::: "memory");

  EpiArgs ea{p.c0, p.c1, p.c2, p.ldc, p.c_gstride, p.aux0, p.aux1, p.N, p.M};
  Work wo = w;
  if (TR::kKRAGGED) wo.row0 = 0;  // outputs of wgrad are indexed by m0 + row
  constexpr int CH = epi_chunk<MODE, NW>(TL::STAGE, S);
  constexpr int NCS = epi_ncs<MODE, NW>(TL::STAGE, S);
  constexpr int REG = epi_region_bytes<MODE>(CH, NCS);
  constexpr int PER = TL::STAGE / REG;
  static_assert(S * PER >= NW, "epilogue staging regions do not fit the stage buffers");
  const int sel = wave / PER;
  LDS_AS unsigned char* wbuf =
      (sel == 0 ? (LDS_AS unsigned char*)lds0 : sel == 1 ? (LDS_AS unsigned char*)lds1
                                                         : (LDS_AS unsigned char*)lds2) +
      (wave % PER) * REG;
  store_tile<MODE, BM, SM, true, CH, NCS>(acc, ea, wo, lane, wm, wn, wbuf);
  }  // tiles of this block
#endif
}

// Padded K start of every expert for the K-ragged GEMMs: kbase[e] =
// sum_{e' < e} roundup(n_e', 128), one block, fixed-order scan (E <= 1024).
__global__ void __launch_bounds__(1024) mx_kbase_kernel(const int32_t* __restrict__ offsets, int E,
                                                        int32_t* __restrict__ kbase) {
  __shared__ int sc[1024];
  const int t = threadIdx.x;
  const int v = t < E ? (offsets[t + 1] - offsets[t] + 127) / 128 * 128 : 0;
  sc[t] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = t >= off ? sc[t - off] : 0;
    __syncthreads();
    sc[t] += add;
    __syncthreads();
  }
  if (t < E) kbase[t] = sc[t] - v;
}

// Tile configurations per mode: rows per tile, stages, waves per block.
#ifndef MX_CFG
#define MX_CFG 256, 2, 8
#endif
#ifndef MX_UP_CFG
#define MX_UP_CFG MX_CFG
#endif
#ifndef MX_DN_CFG
#define MX_DN_CFG MX_CFG
#endif
#ifndef MX_DD_CFG
#define MX_DD_CFG MX_CFG
#endif
#ifndef MX_DU_CFG
#define MX_DU_CFG MX_CFG
#endif
#ifndef MX_WD_CFG
#define MX_WD_CFG MX_CFG
#endif
#ifndef MX_WU_CFG
#define MX_WU_CFG MX_CFG
#endif
template <int BM_, int S_, int NW_>
struct MxCfg {
  static constexpr int BM = BM_, S = S_, NW = NW_;
};
using MxUP = MxCfg<MX_UP_CFG>;
using MxDN = MxCfg<MX_DN_CFG>;
using MxDD = MxCfg<MX_DD_CFG>;
using MxDU = MxCfg<MX_DU_CFG>;
using MxWD = MxCfg<MX_WD_CFG>;
using MxWU = MxCfg<MX_WU_CFG>;

template <int MODE, int BM, int S, int NW>
hipError_t launch_mx(const MxParams& p, int blocks, hipStream_t s) {
  // K-ragged: blocks walk their XCD's cost-balanced tile range.  With at
  // least 16 tiles per CU, one block per CU (the range set-up paid once per
  // CU: 4-7 % faster with 128 experts of 2048 x 1024, uniformly or
  // Zipf-routed); with fewer, four blocks per CU, whose dynamic dispatch
  // evens out skewed tile costs that fixed strides over a few tiles would
  // not (16 Zipf-routed experts of 4096 x 1536: 14 % faster down wgrad).
  if (Traits<MODE>::kKRAGGED) {
    const int cus = moe_host::device_cus();
    blocks = std::min(blocks, (blocks >= 16 * cus ? 1 : 4) * cus);
  }
  blocks = (blocks + 7) / 8 * 8;
  grouped_gemm_mx_kernel<MODE, BM, S, NW><<<blocks, 64 * NW, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------- host side
using namespace moe_host;

// Layout of the MXFP8 workspace of one forward or backward call: byte ranges
// (all 256-byte aligned) for every quantised operand.
namespace {
struct MxLayout {
  size_t total = 0;
  size_t put(size_t bytes) {
    const size_t at = total;
    total += (bytes + 255) & ~(size_t)255;
    return at;
  }
};
int kpad_ld_for(int R, int E) { return (int)((mx_kpad_bound(R, E) + 127) / 128 * 128); }
}  // namespace

size_t moe_internal_mx_fwd_bytes(int E, int R, int d, int F) {
  MxLayout L;
  L.put((size_t)R * d);            // xp codes
  L.put((size_t)R * d / 32);       // xp scales
  L.put((size_t)E * d * F * 2);    // wg, wu codes (K = d, transposed)
  L.put((size_t)E * d * F * 2 / 32);
  L.put((size_t)R * F);            // h codes
  L.put((size_t)R * F / 32);
  L.put((size_t)E * F * d);        // wd codes (K = F, transposed)
  L.put((size_t)E * F * d / 32);
  return L.total;
}

size_t moe_internal_mx_bwd_bytes(int E, int R, int d, int F) {
  const size_t kp = (size_t)kpad_ld_for(R, E);
  MxLayout L;
  L.put((size_t)R * d);            // dyp codes (rowwise along d)
  L.put((size_t)R * d / 32);
  L.put((size_t)E * F * d);        // wd rowwise along d
  L.put((size_t)E * F * d / 32);
  L.put((size_t)R * F * 2);        // dg, du rowwise along F
  L.put((size_t)R * F * 2 / 32);
  L.put((size_t)E * d * F * 2);    // wg, wu rowwise along F
  L.put((size_t)E * d * F * 2 / 32);
  L.put((size_t)d * kp);           // xp^T per-expert column blocks
  L.put((size_t)d * kp / 32);
  L.put((size_t)F * kp * 3);       // dg^T, du^T, h^T
  L.put((size_t)F * kp * 3 / 32);
  L.put((size_t)d * kp);           // dyp^T
  L.put((size_t)d * kp / 32);
  L.put((size_t)(E + 1) * 4);      // padded K start of every expert
  return L.total;
}

// Weight pack: the three expert weights in the two layouts the MXFP8 GEMMs
// read, each region 256-byte aligned.  Forward (blocks along each expert
// matrix's rows, the forward GEMMs' K; transposed): Wg, Wu codes [F][E*d],
// Wd codes [d][E*F].  Backward (blocks along the columns, the data-gradient
// GEMMs' K): Wg, Wu codes [E*d][F], Wd codes [E*F][d].  Scales follow their
// codes ([..][../32]).  base null: sizes only.
size_t moe_internal_mx_pack_layout(int E, int d, int F, uint8_t* base, MxWeights* w) {
  MxLayout L;
  const size_t wgu = (size_t)E * d * F;
  const size_t o[12] = {L.put(wgu), L.put(wgu / 32), L.put(wgu), L.put(wgu / 32), L.put(wgu), L.put(wgu / 32),
                        L.put(wgu), L.put(wgu / 32), L.put(wgu), L.put(wgu / 32), L.put(wgu), L.put(wgu / 32)};
  if (base && w) {
    w->fgq = base + o[0]; w->fgs = base + o[1];
    w->fuq = base + o[2]; w->fus = base + o[3];
    w->fdq = base + o[4]; w->fds = base + o[5];
    w->bgq = base + o[6]; w->bgs = base + o[7];
    w->buq = base + o[8]; w->bus = base + o[9];
    w->bdq = base + o[10]; w->bds = base + o[11];
  }
  return L.total;
}

// Each weight read once, both layouts written (mx_quantize_both, one group of
// rows per expert matrix).
moe_status moe_internal_mx_quantize_weights(moe_ctx* ctx, const bf16_t* wg, const bf16_t* wu,
                                            const bf16_t* wd, int E, int d, int F, uint8_t* pack) {
  MxWeights w;
  moe_internal_mx_pack_layout(E, d, F, pack, &w);
  hipStream_t s = ctx->stream;
  moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
  hipError_t e = mx_quantize_both(wg, E * d, F, nullptr, d, E, (uint8_t*)w.fgq, (uint8_t*)w.fgs, E * d,
                                  (uint8_t*)w.bgq, (uint8_t*)w.bgs, s);
  if (e == hipSuccess)
    e = mx_quantize_both(wu, E * d, F, nullptr, d, E, (uint8_t*)w.fuq, (uint8_t*)w.fus, E * d,
                         (uint8_t*)w.buq, (uint8_t*)w.bus, s);
  if (e == hipSuccess)
    e = mx_quantize_both(wd, E * F, d, nullptr, F, E, (uint8_t*)w.fdq, (uint8_t*)w.fds, E * F,
                         (uint8_t*)w.bdq, (uint8_t*)w.bds, s);
  if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX quantise weights: %s", hipGetErrorString(e));
  return MOE_OK;
}

// xq_in/xs_in: Xp already quantised rowwise (quantise-on-permute); when
// null, Xp is quantised here from the bf16 xp.  pw: the weights already
// quantised (a weight pack); when null, they are quantised here.
moe_status moe_internal_ffn_fwd_mx(moe_ctx* ctx, const bf16_t* xp, const uint8_t* xq_in,
                                   const uint8_t* xs_in, const bf16_t* wg, const bf16_t* wu,
                                   const bf16_t* wd, const MxWeights* pw, const int32_t* offsets,
                                   int E, int R, int d, int F, bf16_t* g, bf16_t* u, bf16_t* h,
                                   bf16_t* yp) {
  const size_t need = moe_internal_mx_fwd_bytes(E, R, d, F);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "MXFP8 forward: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  uint8_t* ws = (uint8_t*)ctx->ws;
  MxLayout L;
  const uint8_t* xq = ws + L.put((size_t)R * d);
  const uint8_t* xs = ws + L.put((size_t)R * d / 32);
  uint8_t* wgq = ws + L.put((size_t)E * d * F * 2);
  uint8_t* wgs = ws + L.put((size_t)E * d * F * 2 / 32);
  uint8_t* wuq = wgq + (size_t)E * d * F;
  uint8_t* wus = wgs + (size_t)E * d * F / 32;
  uint8_t* hq = ws + L.put((size_t)R * F);
  uint8_t* hs = ws + L.put((size_t)R * F / 32);
  uint8_t* wdq = ws + L.put((size_t)E * F * d);
  uint8_t* wds = ws + L.put((size_t)E * F * d / 32);
  hipStream_t s = ctx->stream;
  hipError_t e;
  {
    moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
    // activations along d; weights along d per column, transposed to [F][E*d]
    if (xq_in) {
      xq = xq_in;
      xs = xs_in;
      e = hipSuccess;
    } else {
      e = mx_quantize_rows(xp, R, d, (uint8_t*)xq, (uint8_t*)xs, s);
    }
    if (pw) {
      wgq = (uint8_t*)pw->fgq; wgs = (uint8_t*)pw->fgs;
      wuq = (uint8_t*)pw->fuq; wus = (uint8_t*)pw->fus;
      wdq = (uint8_t*)pw->fdq; wds = (uint8_t*)pw->fds;
    } else {
      if (e == hipSuccess) e = mx_quantize_cols(wg, E * d, F, nullptr, d, E, wgq, wgs, E * d, s);
      if (e == hipSuccess) e = mx_quantize_cols(wu, E * d, F, nullptr, d, E, wuq, wus, E * d, s);
      if (e == hipSuccess && wd) e = mx_quantize_cols(wd, E * F, d, nullptr, F, E, wdq, wds, E * F, s);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX quantise: %s", hipGetErrorString(e));
  }
  {
    MxParams p{};
    p.a0 = xq; p.sa0 = xs; p.lda = d;
    p.b0 = wgq; p.sb0 = wgs; p.b1 = wuq; p.sb1 = wus; p.ldb = E * d; p.b_k_e = d;
    p.c0 = g; p.c1 = u; p.c2 = h; p.ldc = F;
    p.offsets = offsets; p.E = E; p.N = F; p.K = d; p.kseg = d;
    p.ntiles = (F + 127) / 128;
    moe_prof_scope ps(ctx, MOE_K_GEMM_UP);
    e = launch_mx<FWD_UP, MxUP::BM, MxUP::S, MxUP::NW>(p, (R / MxUP::BM + E) * p.ntiles, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX gate/up: %s", hipGetErrorString(e));
  }
  if (yp == nullptr) return MOE_OK;  // gate/up alone (recompute)
  {
    moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
    e = mx_quantize_rows(h, R, F, hq, hs, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX quantise h: %s", hipGetErrorString(e));
  }
  {
    MxParams p{};
    p.a0 = hq; p.sa0 = hs; p.lda = F;
    p.b0 = wdq; p.sb0 = wds; p.ldb = E * F; p.b_k_e = F;
    p.c0 = yp; p.ldc = d;
    p.offsets = offsets; p.E = E; p.N = d; p.K = F; p.kseg = F;
    p.ntiles = (d + BN - 1) / BN;
    moe_prof_scope ps(ctx, MOE_K_GEMM_DOWN);
    e = launch_mx<FWD_DOWN, MxDN::BM, MxDN::S, MxDN::NW>(p, (R / MxDN::BM + E) * p.ntiles, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX down: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

size_t moe_internal_wgrads_bf16_bytes(int E, int R, int d, int F);  // gemm_bf16.hip
moe_status moe_internal_wgrads_bf16(moe_ctx* ctx, const bf16_t* xp, const int32_t* offsets,
                                    const bf16_t* dg, const bf16_t* du, const bf16_t* h,
                                    const bf16_t* dyp, int E, int R, int d, int F, bf16_t* dwg,
                                    bf16_t* dwu, bf16_t* dwd, void* ws);

// wgrad_bf16: MXFP8 on the two data-gradient GEMMs only; dyp, dg and du are
// quantised rowwise alone (no column layouts, no Xp or H columns) and the
// three weight gradients run on the bf16 operands (the bf16 backward's
// launches, their workspace after the MXFP8 layout).
moe_status moe_internal_ffn_bwd_mx(moe_ctx* ctx, const bf16_t* xp, const bf16_t* wg,
                                   const bf16_t* wu, const bf16_t* wd, const MxWeights* pw,
                                   const int32_t* offsets, const bf16_t* g, const bf16_t* u,
                                   const bf16_t* h, const bf16_t* dyp, int E, int R, int d, int F,
                                   bf16_t* dg, bf16_t* du, bf16_t* dxp, bf16_t* dwg, bf16_t* dwu,
                                   bf16_t* dwd, bool wgrad_bf16) {
  const size_t mx_need = moe_internal_mx_bwd_bytes(E, R, d, F);
  const size_t need = mx_need + (wgrad_bf16 ? moe_internal_wgrads_bf16_bytes(E, R, d, F) : 0);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "MXFP8 backward: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  const int kp = kpad_ld_for(R, E);
  uint8_t* ws = (uint8_t*)ctx->ws;
  MxLayout L;
  uint8_t* dyq = ws + L.put((size_t)R * d);
  uint8_t* dys = ws + L.put((size_t)R * d / 32);
  uint8_t* wdq = ws + L.put((size_t)E * F * d);
  uint8_t* wds = ws + L.put((size_t)E * F * d / 32);
  uint8_t* dgq = ws + L.put((size_t)R * F * 2);
  uint8_t* dgs = ws + L.put((size_t)R * F * 2 / 32);
  uint8_t* duq = dgq + (size_t)R * F;
  uint8_t* dus = dgs + (size_t)R * F / 32;
  uint8_t* wgq = ws + L.put((size_t)E * d * F * 2);
  uint8_t* wgs = ws + L.put((size_t)E * d * F * 2 / 32);
  uint8_t* wuq = wgq + (size_t)E * d * F;
  uint8_t* wus = wgs + (size_t)E * d * F / 32;
  uint8_t* xtq = ws + L.put((size_t)d * kp);
  uint8_t* xts = ws + L.put((size_t)d * kp / 32);
  uint8_t* gtq = ws + L.put((size_t)F * kp * 3);
  uint8_t* gts = ws + L.put((size_t)F * kp * 3 / 32);
  uint8_t* utq = gtq + (size_t)F * kp;
  uint8_t* uts = gts + (size_t)F * kp / 32;
  uint8_t* htq = utq + (size_t)F * kp;
  uint8_t* hts = uts + (size_t)F * kp / 32;
  uint8_t* ytq = ws + L.put((size_t)d * kp);
  uint8_t* yts = ws + L.put((size_t)d * kp / 32);
  int32_t* kbase = (int32_t*)(ws + L.put((size_t)(E + 1) * 4));
  hipStream_t s = ctx->stream;
  hipError_t e;
  {
    moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
    // dyp in both layouts from one read (rows for the down dgrad, expert
    // column blocks for the down wgrad)
    if (wgrad_bf16)
      e = mx_quantize_rows(dyp, R, d, dyq, dys, s);
    else
      e = mx_quantize_both(dyp, R, d, offsets, 0, E, ytq, yts, kp, dyq, dys, s);
    if (pw) {
      wdq = (uint8_t*)pw->bdq; wds = (uint8_t*)pw->bds;
      wgq = (uint8_t*)pw->bgq; wgs = (uint8_t*)pw->bgs;
      wuq = (uint8_t*)pw->buq; wus = (uint8_t*)pw->bus;
    } else {
      if (e == hipSuccess) e = mx_quantize_rows(wd, E * F, d, wdq, wds, s);
      if (e == hipSuccess) e = mx_quantize_rows(wg, E * d, F, wgq, wgs, s);
      if (e == hipSuccess) e = mx_quantize_rows(wu, E * d, F, wuq, wus, s);
    }
    if (!wgrad_bf16) {
      if (e == hipSuccess) e = mx_quantize_cols(xp, R, d, offsets, 0, E, xtq, xts, kp, s);
      if (e == hipSuccess) e = mx_quantize_cols(h, R, F, offsets, 0, E, htq, hts, kp, s);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX quantise: %s", hipGetErrorString(e));
  }
  if (!wgrad_bf16) mx_kbase_kernel<<<1, 1024, 0, s>>>(offsets, E, kbase);
  if (R > 0) {
    MxParams p{};
    p.a0 = dyq; p.sa0 = dys; p.lda = d;
    p.b0 = wdq; p.sb0 = wds; p.ldb = d; p.b_row_e = F;
    p.c0 = dg; p.c1 = du; p.ldc = F; p.aux0 = g; p.aux1 = u;
    p.offsets = offsets; p.E = E; p.N = F; p.K = d; p.kseg = d;
    p.ntiles = (F + BN - 1) / BN;
    moe_prof_scope ps(ctx, MOE_K_GEMM_DGRAD_DOWN);
    e = launch_mx<DGRAD_DOWN, MxDD::BM, MxDD::S, MxDD::NW>(p, (R / MxDD::BM + E) * p.ntiles, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX down dgrad: %s", hipGetErrorString(e));
  }
  if (!wgrad_bf16) {
    MxParams p{};
    p.a0 = htq; p.sa0 = hts; p.lda = kp;
    p.b0 = ytq; p.sb0 = yts; p.ldb = kp;
    p.c0 = dwd; p.ldc = d; p.c_gstride = (long long)F * d;
    p.offsets = offsets; p.E = E; p.M = F; p.N = d; p.kbase = kbase;
    p.ntiles = (d + BN - 1) / BN;
    p.mtiles = (F + MxWD::BM - 1) / MxWD::BM;
    moe_prof_scope ps(ctx, MOE_K_GEMM_WGRAD_DOWN);
    e = launch_mx<WGRAD_DOWN, MxWD::BM, MxWD::S, MxWD::NW>(p, E * p.ntiles * p.mtiles, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX down wgrad: %s", hipGetErrorString(e));
  }
  {
    moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
    if (wgrad_bf16) {
      e = mx_quantize_rows(dg, R, F, dgq, dgs, s);
      if (e == hipSuccess) e = mx_quantize_rows(du, R, F, duq, dus, s);
    } else {
      e = mx_quantize_both(dg, R, F, offsets, 0, E, gtq, gts, kp, dgq, dgs, s);
      if (e == hipSuccess) e = mx_quantize_both(du, R, F, offsets, 0, E, utq, uts, kp, duq, dus, s);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX quantise dg/du: %s", hipGetErrorString(e));
  }
  if (R > 0) {
    MxParams p{};
    p.a0 = dgq; p.sa0 = dgs; p.a1 = duq; p.sa1 = dus; p.lda = F;
    p.b0 = wgq; p.sb0 = wgs; p.b1 = wuq; p.sb1 = wus; p.ldb = F; p.b_row_e = d;
    p.c0 = dxp; p.ldc = d;
    p.offsets = offsets; p.E = E; p.N = d; p.K = 2 * F; p.kseg = F;
    p.ntiles = (d + BN - 1) / BN;
    moe_prof_scope ps(ctx, MOE_K_GEMM_DGRAD_UP);
    e = launch_mx<DGRAD_UP, MxDU::BM, MxDU::S, MxDU::NW>(p, (R / MxDU::BM + E) * p.ntiles, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX gate/up dgrad: %s", hipGetErrorString(e));
  }
  if (wgrad_bf16)
    return moe_internal_wgrads_bf16(ctx, xp, offsets, dg, du, h, dyp, E, R, d, F, dwg, dwu, dwd, ws + mx_need);
  {
    MxParams p{};
    p.a0 = xtq; p.sa0 = xts; p.lda = kp;
    p.b0 = gtq; p.sb0 = gts; p.b1 = utq; p.sb1 = uts; p.ldb = kp;
    p.c0 = dwg; p.c1 = dwu; p.ldc = F; p.c_gstride = (long long)d * F;
    p.offsets = offsets; p.E = E; p.M = d; p.N = F; p.kbase = kbase;
    p.ntiles = (F + 127) / 128;
    p.mtiles = (d + MxWU::BM - 1) / MxWU::BM;
    moe_prof_scope ps(ctx, MOE_K_GEMM_WGRAD_UP);
    e = launch_mx<WGRAD_UP, MxWU::BM, MxWU::S, MxWU::NW>(p, E * p.ntiles * p.mtiles, s);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "MX gate/up wgrad: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}
