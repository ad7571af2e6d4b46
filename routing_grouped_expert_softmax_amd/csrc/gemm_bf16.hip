// gemm_bf16.hip — device-scheduled grouped GEMM for the SwiGLU experts on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Pages: many small per-expert GEMMs are merged into one grouped GEMM so the
// GPU is fed ([P1] 核心特点 二, Grouped GEMM); it is scheduled on the device from
// GPU-resident routing metadata, with no host synchronisation ([P1] 二); the
// layer is dropless ([P3]).  The pages' kernel is prior art for another GPU;
// this one is written for CDNA4:
//
//  * Block tile BM x 256 x BK: NW waves in an (NW/2) x 2 grid, each wave a
//    64 x 128 sub-tile of 32x32 MFMA tiles (128 accumulator registers, at
//    most 256 registers per wave).  The forward GEMMs and the wgrads run
//    128 x 256 x 32 tiles, four waves, two resident blocks per CU; the dgrads
//    run 288 x 256 x 64 tiles, eight waves, one block per CU: 256 rows as
//    above plus a 32-row strip of one 32x32 MFMA tile per wave (see the tile
//    configurations below).
//  * Tiles move HBM -> LDS with buffer loads that write LDS directly (16 bytes
//    per lane), S stages deep, one static LDS array per stage, explicit vmcnt
//    waits and a fence-free barrier; no VGPR staging, no VALU transposes.
//  * K-contiguous operands (activations in the forward pass and dgrad, weight
//    rows in dgrad) feed the MFMA with ds_read_b128; M/N-contiguous operands
//    (weights in the forward pass, both operands in wgrad) with two
//    ds_read_b64_tr_b16 (hardware transpose) per fragment.  Both LDS layouts
//    are swizzled so the direct-load writes and the fragment reads are free of
//    bank conflicts (measured: zero).
//  * The MFMA operands are swapped (B fragment as the A operand) so each lane
//    ends with four consecutive output columns per register group: 8-byte
//    stores, with the SwiGLU forward/backward fused into the epilogue.
//  * Scheduling: M-ragged launches (forward, dgrad) size the grid from the host
//    bound sum_e ceil(n_e/BM) <= R/BM + E; every block scans the per-expert
//    counts (from `offsets`, read on the device) to find its (expert, m-tile,
//    n-tile); blocks past the real total exit.  Logical tiles are handed to
//    the 8 XCDs in contiguous ranges (block b runs on XCD b % 8), and within an
//    expert the m-tiles sharing one weight tile are consecutive, so they meet
//    in the same L2.  K-ragged launches (wgrad) have a fixed tile grid per
//    expert and loop over that expert's own rows; an expert with no rows
//    writes zeros.  Their XCD ranges balance K steps, not tile counts (with
//    skewed routing a hot expert's tiles would pile onto one XCD): the down
//    dgrad plans them for both weight gradients in eight extra blocks.
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

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

struct Params {
  const bf16_t* a0;  // A operand (segment 0)
  const bf16_t* a1;  // A operand, second K segment (DGRAD_UP)
  int lda;
  const bf16_t* b0;  // B operand (or first of the pair)
  const bf16_t* b1;  // second B (dual) or second K segment (DGRAD_UP)
  int ldb;
  long long b_gstride;  // per-expert stride of B (weights); 0 if B is per-row data
  void* c0;
  void* c1;
  void* c2;
  int ldc;
  long long c_gstride;  // per-expert stride of C (wgrad outputs)
  const bf16_t* aux0;   // saved g (DGRAD_DOWN)
  const bf16_t* aux1;   // saved u (DGRAD_DOWN)
  const int32_t* offsets;
  int E;
  int M;      // fixed M (K-ragged: output rows; ROUTER: T)
  int N;      // columns per output matrix
  int K;      // fixed K (M-ragged)
  int kseg;   // K of segment 0 (DGRAD_UP), else K
  int ntiles;  // tiles along N
  int mtiles;  // tiles along M (K-ragged)
  int part;    // K-ragged: store exact fp32 split-K partials instead of bf16
  // DGRAD_UP, optional router term: row r of expert e gets
  // rdl[r] * rw[:, e] (rw is the [N, E] router weight matrix)
  const float* rdl;
  const bf16_t* rw;
  // K-ragged: per-XCD tile ranges [first, end) as 8 pairs; nullptr = equal
  // tile counts per XCD
  const int32_t* xr;
  // DGRAD_DOWN: block 0 also writes the ranges of the two weight gradients
  // that follow (xr_pe0 / xr_pe1 tiles per group)
  int32_t* xr_out0;
  int32_t* xr_out1;
  int xr_pe0, xr_pe1;
};

// K step of the weight gradients, for their XCD range plans
constexpr int kWgradBK = 32;

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

// ---------------------------------------------------------------- LDS layouts
// K-contiguous tile: groups of 8 rows, each group 16*BK bytes laid out as
// [16-deep K slice][row % 8][32 bytes], the two 16-byte halves of a row
// swapped when bit 3 of the row is set.  One 1 KiB load instruction fills
// 1024 / (16*BK) whole groups (8 full row segments of HBM each); the 16 lanes
// of one LDS pass (16 consecutive rows, same half) hit 16 distinct bank
// slots; a fragment address is one per-lane base plus a compile-time offset
// per row block and slice.
__device__ __forceinline__ int kc_half(int row, int h) { return h ^ ((row >> 3) & 1); }
// M/N-contiguous tile ([64 k][cols], 256- or 512-byte rows): the 16-byte
// chunk index is XOR-ed with 4*(k & 3), so a transposing fragment read
// (4 k rows x 32 bytes per 16 lanes, two groups side by side) covers every
// bank slot once per 32 lanes.
__device__ __forceinline__ int swz_mn(int k) { return (k & 3) << 2; }

// Tile geometry of one pipeline stage.
// BM is a multiple of 64 (BMAIN rows, NW/2 waves down) plus an optional
// 32-row strip (XR = 32): the strip's 32 x 256 outputs are spread over the NW
// waves as one 32x32 MFMA tile each, so an expert of up to 2 * BM rows takes
// two row tiles where 256-row tiles would need a third, nearly empty one.
template <int MODE, int BM, int BK, int NW = 4>
struct Tile {
  using TR = Traits<MODE>;
  static constexpr int XR = BM % 64;        // rows of the extra strip (0 or 32)
  static constexpr int BMAIN = BM - XR;
  static constexpr int WM = BMAIN / (NW / 2);  // wave tile rows (M): NW/2 waves down, 2 across
  static constexpr int SM = WM / 32;  // 32-row subtiles per wave
  static constexpr int GROUP = 16 * BK;     // bytes of one 8-row K-contiguous group
  static constexpr int SLICES = BK / 16;    // 16-deep K slices per stage
  static constexpr int GPI = 1024 / GROUP;  // groups filled by one 1 KiB load
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INST = BMAIN * BK * 2 / 1024 / NW;  // 1 KiB direct loads per wave
  static constexpr int XA_INST = XR * BK * 2 / 1024;  // strip loads: one each for waves 0..XA_INST-1
  static constexpr int B_INST = B_BYTES / 1024 / NW;
  static constexpr int A_PITCH = TR::kA_KCONTIG ? 128 : BM * 2;  // LDS row pitch (bytes)
  // B: K-contiguous [256][64]; N-contiguous [64][256]; dual: two [64][128]
  static constexpr int B_PITCH = TR::kB_KCONTIG ? 128 : (TR::kDUAL ? 256 : 512);
};

// NF: row-ragged tiles of one expert in m-major order (its n-tiles
// consecutive) instead of n-major (its m-tiles consecutive).
template <int MODE, int BM, int S, int BK, int OCC, int NW, bool NF = false>
__global__ void __launch_bounds__(64 * NW, OCC) grouped_gemm_kernel(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using TR = Traits<MODE>;
  using TL = Tile<MODE, BM, BK, NW>;
  constexpr int SM = TL::SM;
  static_assert(TL::XR == 0 || (TL::XR == 32 && S == 2 && NW == 8 && TL::GPI == 1 && TR::kA_KCONTIG &&
                                TR::kB_KCONTIG && !TR::kKRAGGED && !TR::kDUAL && TL::XA_INST <= NW),
                "the 32-row strip is built for the eight-wave, two-stage, K-contiguous dgrad tiles");
  // One LDS array per pipeline stage: distinct objects let the compiler see
  // that fragment reads of one stage never alias the loads landing in another.
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[TL::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds2[S > 2 ? TL::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char lds3[S > 3 ? TL::STAGE : 16];
  __shared__ int sh[kThreads + 4];
  // router term (DGRAD_UP): the tile's W_r column and its rows' logit gradients
  __shared__ float rcol[MODE == DGRAD_UP ? BN : 1];
  __shared__ float rrow[MODE == DGRAD_UP ? BM : 1];

  const int tid = threadIdx.x;
  const int lane0 = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // With a plan (DGRAD_DOWN, xr_out0 set) the last eight blocks of the grid
  // plan instead of computing: the one on XCD x writes that XCD's tile ranges
  // for the two weight gradients launched after this kernel (they read them
  // in stream order) and exits.  Dispatched last, the plan blocks run while
  // the final tiles finish (at the front of the grid they delayed eight
  // compute units' first tiles).
  int bid = blockIdx.x, nblk = gridDim.x;
  if constexpr (MODE == DGRAD_DOWN) {
    if (p.xr_out0 != nullptr) {
      nblk -= 8;
      if (bid >= nblk) {
        bid &= 7;
        if (wv == 0) {
          int f0, f1;
          kragged_xcd_range<kWgradBK>(p.offsets, p.E, p.xr_pe0, bid, f0, f1);
          if (lane0 == 0) {
            p.xr_out0[2 * bid] = f0;
            p.xr_out0[2 * bid + 1] = f1;
          }
          kragged_xcd_range<kWgradBK>(p.offsets, p.E, p.xr_pe1, bid, f0, f1);
          if (lane0 == 0) {
            p.xr_out1[2 * bid] = f0;
            p.xr_out1[2 * bid + 1] = f1;
          }
        }
        return;
      }
    }
  }

  // ---------------------------------------------------------------- work
  // Logical tiles are split into eight contiguous ranges, one per XCD (block
  // b runs on XCD b % 8), so the blocks of one XCD share operands in its L2:
  // equal tile counts for row-ragged launches, cost-balanced ranges for
  // K-ragged ones.  Block b takes tiles first + b / 8, + nslot, ... of its
  // XCD's range.
  MTileSched<BM, NF> ms;
  int first, end;  // this XCD's range of logical tiles
  if (TR::kKRAGGED) {
    // A tile costs as many K steps as its expert has rows: with skewed
    // routing one expert's tiles would pile onto one XCD.  The ranges come
    // precomputed (cost-balanced unless equal tile counts are within 10 % of
    // balanced); blocks of an XCD whose range is longer than its share of
    // the grid walk several tiles.
    const int x = bid & 7;
    if (p.xr != nullptr) {
      first = p.xr[2 * x];
      end = p.xr[2 * x + 1];
    } else {
      const int total = p.E * p.ntiles * p.mtiles;
      const int per_xcd = (total + 7) / 8;
      first = min(x * per_xcd, total);
      end = min(first + per_xcd, total);
    }
  } else {
    int total;
    if (TR::kSINGLE) {
      total = ((p.M + BM - 1) / BM) * p.ntiles;
    } else {
      ms.init(p.E, p.offsets, p.ntiles, sh);
      total = ms.total;
    }
    const int per_xcd = (total + 7) / 8;
    first = (bid & 7) * per_xcd;
    end = min(first + per_xcd, total);
  }
  const int nslot = nblk >> 3;
  const int L0 = first + (bid >> 3);
  for (int L = L0; L < end; L += nslot) {
  // the previous tile's epilogue has finished with the LDS stage buffers
  if (L != L0) lds_barrier();
  // With the strip, registers are short: the lane id is made opaque per tile
  // so lane-derived addresses are recomputed in each tile, not held (and
  // spilled) across the whole tile loop.
  int lane = lane0;
  if constexpr (TL::XR > 0) asm volatile("" : "+v"(lane));
  Work w;
  if (TR::kKRAGGED) {
    // expert-major, then m-tile, then n-tile (n fastest: the blocks of one
    // XCD write neighbouring column ranges of the same output rows)
    const int per_e = p.ntiles * p.mtiles;
    w.e = L / per_e;
    const int r = L % per_e;
    w.nt = r % p.ntiles;
    w.m0 = (r / p.ntiles) * BM;
    w.row0 = p.offsets[w.e];
    w.rows = p.offsets[w.e + 1] - w.row0;
  } else if (TR::kSINGLE) {
    const int mt_total = (p.M + BM - 1) / BM;
    w.e = 0;
    w.nt = L / mt_total;
    w.row0 = (L % mt_total) * BM;
    w.rows = min(BM, p.M - w.row0);
    w.m0 = 0;
  } else {
    ms.lookup(L, p.offsets, sh, w);
  }
  const int nk = TR::kKRAGGED ? (w.rows + BK - 1) / BK : p.K / BK;

  // ---------------------------------------------------------------- sources
  // Raw buffer descriptors whose ranges cover exactly the rows this block may
  // read: rows past a tile's valid rows, past an expert's K rows or past a
  // weight matrix read as zero (the loads below never branch).  Columns past
  // N only feed output columns that are never stored.
  const size_t esz = sizeof(bf16_t);
  rsrc_t rsa0, rsa1, rsb0, rsb1;
  {
    const size_t abytes = (size_t)max(w.rows, 0) * p.lda * esz;
    rsa0 = make_rsrc((void*)(p.a0 + (size_t)w.row0 * p.lda), abytes);
    rsa1 = rsa0;
    if (MODE == DGRAD_UP)
      rsa1 = make_rsrc((void*)(p.a1 + (size_t)w.row0 * p.lda), abytes);
    if (TR::kKRAGGED) {
      const size_t bbytes = (size_t)max(w.rows, 0) * p.ldb * esz;
      rsb0 = make_rsrc((void*)(p.b0 + (size_t)w.row0 * p.ldb), bbytes);
      rsb1 = TR::kDUAL ? make_rsrc((void*)(p.b1 + (size_t)w.row0 * p.ldb), bbytes) : rsb0;
    } else {
      const size_t bbytes = (size_t)(TR::kB_KCONTIG ? p.N : p.K) * p.ldb * esz;
      rsb0 = make_rsrc((void*)(p.b0 + (size_t)w.e * p.b_gstride), bbytes);
      rsb1 = (TR::kDUAL || MODE == DGRAD_UP)
                 ? make_rsrc((void*)(p.b1 + (size_t)w.e * p.b_gstride), bbytes)
                 : rsb0;
    }
  }

  // Per-lane byte offsets of this wave's direct loads (fixed over the K loop;
  // the K advance goes in the scalar offset).  Each load moves 16 bytes per
  // lane into LDS at (instruction base + 16 * lane), so the global side picks
  // the source chunk that belongs at that (swizzled) LDS position.  The
  // swizzle repeats every P instructions of a wave, so load j uses the
  // per-lane offset of load j % P plus a uniform (j / P) * R rows (in the
  // scalar offset): P per-lane values per operand instead of one per load.
  constexpr int A_RPI = 64 / (BM / 8);  // k rows per load, M-contiguous A
  constexpr int PA = TR::kA_KCONTIG ? (TL::GPI == 1 ? 2 : 1) : (A_RPI >= 4 ? 1 : 4 / A_RPI);
  constexpr int RA = TR::kA_KCONTIG ? PA * TL::GPI * 8 : PA * A_RPI;
  constexpr int PB = TR::kB_KCONTIG ? (TL::GPI == 1 ? 2 : 1) : (TR::kDUAL ? 1 : 2);
  constexpr int RB = TR::kB_KCONTIG ? PB * TL::GPI * 8 : 4;
  static_assert(TL::A_INST % PA == 0 && TL::B_INST % PB == 0, "loads per wave come in whole periods");
  static_assert(!TR::kDUAL || TR::kB_KCONTIG || (BK / 4) % TL::B_INST == 0,
                "a wave's loads stay inside one matrix of the pair");
  const int astep = RA * p.lda * (int)esz, bstep = RB * p.ldb * (int)esz;
  int aoff[PA], boff[PB];
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    const int q = wv * TL::A_INST + j;  // 1 KiB instruction index inside the A tile
    if (TR::kA_KCONTIG) {
      // instruction q fills groups q*GPI..; lane = (group, slice, row % 8, half)
      const int kk = (lane >> 4) % TL::SLICES, gi = (lane >> 4) / TL::SLICES;
      const int row = (q * TL::GPI + gi) * 8 + ((lane & 15) >> 1), hp = lane & 1;
      aoff[j] = (row * p.lda + (kk * 2 + kc_half(row, hp)) * 8) * (int)esz;
    } else {
      constexpr int CPR = BM / 8;  // 16-byte chunks per k row
      const int k = (q * 64 + lane) / CPR, pc = (q * 64 + lane) % CPR;
      aoff[j] = (k * p.lda + w.m0 + ((pc ^ swz_mn(k)) << 3)) * (int)esz;
    }
  }
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const int q = wv * TL::B_INST + j;
    if (TR::kB_KCONTIG) {
      const int kk = (lane >> 4) % TL::SLICES, gi = (lane >> 4) / TL::SLICES;
      const int n = (q * TL::GPI + gi) * 8 + ((lane & 15) >> 1), hp = lane & 1;
      boff[j] = ((w.nt * BN + n) * p.ldb + (kk * 2 + kc_half(n, hp)) * 8) * (int)esz;
    } else if (TR::kDUAL) {
      // two sub-tiles of [BK k][128 n]: the first BK/4 instructions fill
      // matrix 0 (the lower half of the waves), the rest matrix 1
      const int qq = q % (BK / 4);
      const int k = qq * 4 + (lane >> 4), pc = lane & 15;
      boff[j] = (k * p.ldb + w.nt * 128 + ((pc ^ swz_mn(k)) << 3)) * (int)esz;
    } else {
      const int k = q * 2 + (lane >> 5), pc = lane & 31;
      boff[j] = (k * p.ldb + w.nt * BN + ((pc ^ swz_mn(k)) << 3)) * (int)esz;
    }
  }
  // The strip's A rows (BMAIN..BM-1): 1 KiB instruction A_INST * NW + wave,
  // one for each of the first XA_INST waves, same group layout as the rest.
  int aoffx = 0;
  if constexpr (TL::XR > 0) {
    const int q = TL::A_INST * NW + wv;
    const int kk = (lane >> 4) % TL::SLICES;
    const int row = q * 8 + ((lane & 15) >> 1), hp = lane & 1;
    aoffx = (row * p.lda + (kk * 2 + kc_half(row, hp)) * 8) * (int)esz;
  }

  // Issue the direct loads of K step kt into stage buffer `st`.
  auto stage_ptr = [&](auto st) -> LDS_AS unsigned char* {
    constexpr int ST = decltype(st)::value;
    if constexpr (ST == 0) return (LDS_AS unsigned char*)lds0;
    else if constexpr (ST == 1) return (LDS_AS unsigned char*)lds1;
    else if constexpr (ST == 2) return (LDS_AS unsigned char*)lds2;
    else return (LDS_AS unsigned char*)lds3;
  };
  auto issue = [&](int kt, auto st) {
    const int k0 = kt * BK;
    LDS_AS unsigned char* base = stage_ptr(st);
    // A
    {
      rsrc_t r = rsa0;
      int soff;
      if (TR::kA_KCONTIG) {
        int kk = k0;
        if (MODE == DGRAD_UP && k0 >= p.kseg) {
          r = rsa1;
          kk = k0 - p.kseg;
        }
        soff = kk * (int)esz;
      } else {
        soff = k0 * p.lda * (int)esz;
      }
#pragma unroll
      for (int j = 0; j < TL::A_INST; ++j)
        dma16(r, (LDS_AS void*)(base + (wv * TL::A_INST + j) * 1024), aoff[j % PA],
              soff + (j / PA) * astep);
      if constexpr (TL::XR > 0) {
        if (wv < TL::XA_INST)
          dma16(r, (LDS_AS void*)(base + (TL::A_INST * NW + wv) * 1024), aoffx, soff);
      }
    }
    // B
    {
      LDS_AS unsigned char* bbase = base + TL::A_BYTES;
      rsrc_t r = rsb0;
      int soff;
      if (TR::kB_KCONTIG) {
        int kk = k0;
        if (MODE == DGRAD_UP && k0 >= p.kseg) {
          r = rsb1;
          kk = k0 - p.kseg;
        }
        soff = kk * (int)esz;
      } else {
        soff = k0 * p.ldb * (int)esz;
        if (TR::kDUAL && wv >= NW / 2) r = rsb1;  // the upper half of the waves loads the second matrix
      }
#pragma unroll
      for (int j = 0; j < TL::B_INST; ++j)
        dma16(r, (LDS_AS void*)(bbase + (wv * TL::B_INST + j) * 1024), boff[j % PB],
              soff + (j / PB) * bstep);
    }
  };

  // ---------------------------------------------------------------- fragments
  // K-contiguous tile: lane reads row (row0 + lane & 31), half (lane >> 5) of
  // slice kk.  The per-lane part is computed once; row0 (a multiple of 32)
  // and kk fold into the instruction's immediate offset.
  const int kc_lane = ((lane & 31) >> 3) * TL::GROUP + (lane & 7) * 32 +
                      (kc_half(lane & 31, lane >> 5) << 4);
  auto frag_kc = [&](const LDS_AS unsigned char* t, int row0, int kk) -> bf16x8 {
    return *(const LDS_AS bf16x8*)(t + (row0 >> 3) * TL::GROUP + kk * 256 + kc_lane);
  };
  // M/N-contiguous tile: two transposing 8-byte reads give each lane 8
  // consecutive k of column (col0 + lane & 31): in each 16-lane group, lane i
  // receives element i%4 of the reads of lanes i/4 + 4j, so lane a + 4b
  // addresses row 8*half + 4r + b, columns col0 + 16*group + 4a.  The k of a
  // lane is kk*16 + 8*half + 4r + b, so the swizzle depends on b only and kk,
  // r fold into the immediate offset.
  const int mn_b = (lane & 15) >> 2, mn_g = (lane >> 4) & 1, mn_half = lane >> 5;
  const int mn_x = 2 * mn_g + ((lane & 3) >> 1);   // chunk within the 32-column group
  const int mn_sub = (lane & 1) * 8;               // 8-byte half of the chunk
  auto frag_mn = [&](const LDS_AS unsigned char* t, int pitch, int col0, int kk) -> bf16x8 {
    // (col0/8 + x) ^ 4*b with col0 a multiple of 32: bits 2.. come from col0
    const int chunk = ((col0 >> 3) ^ swz_mn(mn_b)) + mn_x;
    const LDS_AS unsigned char* a = t + (8 * mn_half + mn_b) * pitch + (chunk << 4) + mn_sub;
    bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(a + (kk * 16) * pitch));
    bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(a + (kk * 16 + 4) * pitch));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 acc[SM][4];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // the wave's 32x32 tile of the strip: rows BMAIN.., columns wn*128 + wm*32..
  f32x16 accx[1][1];
#pragma unroll
  for (int r = 0; r < 16; ++r) accx[0][0][r] = 0.f;

  // Fragments of one 16-deep K slice.
  struct Frags {
    bf16x8 xb[4], ya[SM], xbx, yx;
  };
  // 32-row subtiles of this wave that hold at least one valid row: fewer
  // than SM only in an expert's last row tile, whose empty subtiles then
  // skip their fragment reads and MFMAs (wave-uniform branches, in a second
  // copy of the loop so full tiles run branch-free).
  const int nvsm = TR::kKRAGGED ? SM
                                : max(0, min(SM, (w.rows - (wv >> 1) * TL::WM + 31) / 32));
  auto load_frags = [&](const LDS_AS unsigned char* As, int kk, Frags& f, auto full) {
    const LDS_AS unsigned char* Bs = As + TL::A_BYTES;
    if (!decltype(full)::value && nvsm == 0) return;
#pragma unroll
    for (int sn = 0; sn < 4; ++sn) {
      if (TR::kB_KCONTIG) {
        f.xb[sn] = frag_kc(Bs, wn * 128 + sn * 32, kk);
      } else if (TR::kDUAL) {
        // subtiles 0,1: matrix 0 columns wn*64 + ..; 2,3: matrix 1, same columns
        f.xb[sn] = frag_mn(Bs + (sn >> 1) * (BK * 256), 256, wn * 64 + (sn & 1) * 32, kk);
      } else {
        f.xb[sn] = frag_mn(Bs, 512, wn * 128 + sn * 32, kk);
      }
    }
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
      if (!decltype(full)::value && sm >= nvsm) continue;
      if (TR::kA_KCONTIG)
        f.ya[sm] = frag_kc(As, wm * TL::WM + sm * 32, kk);
      else
        f.ya[sm] = frag_mn(As, TL::A_PITCH, wm * TL::WM + sm * 32, kk);
    }
    if constexpr (TL::XR > 0 && decltype(full)::value == 2) {
      f.yx = frag_kc(As, TL::BMAIN, kk);
      f.xbx = frag_kc(Bs, wn * 128 + wm * 32, kk);
    }
  };
  auto mma = [&](const Frags& f, auto full) {
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
      if (!decltype(full)::value && sm >= nvsm) continue;
#pragma unroll
      for (int sn = 0; sn < 4; ++sn)
        acc[sm][sn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.xb[sn], f.ya[sm], acc[sm][sn], 0, 0, 0);
    }
    if constexpr (TL::XR > 0 && decltype(full)::value == 2)
      accx[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.xbx, f.yx, accx[0][0], 0, 0, 0);
  };

  // One stage: the fragments of slice kk+1 are read while the MFMAs of slice
  // kk run (the compiler interleaves the two).
  auto compute = [&](auto st, auto full) {
    const LDS_AS unsigned char* As = stage_ptr(st);
    Frags f0, f1;
    load_frags(As, 0, f0, full);
    load_frags(As, 1, f1, full);
    mma(f0, full);
    if constexpr (BK == 64) {
      load_frags(As, 2, f0, full);
      mma(f1, full);
      load_frags(As, 3, f1, full);
      mma(f0, full);
    }
    mma(f1, full);
  };


  // ---------------------------------------------------------------- main loop
  // S-stage pipeline: at the top of step kt the wave waits for its own loads
  // of stage kt (later stages may stay in flight), a barrier makes every
  // wave's loads visible and frees the buffer read in step kt-1, the loads of
  // step kt+S-1 go into that buffer, then step kt is computed.
  constexpr int LPS = TL::A_INST + TL::B_INST;  // direct loads per wave per stage
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // Router term (DGRAD_UP): its two small loads go out before the first
  // stage's and land in LDS before the first K step's barrier (the wait the
  // compiler puts before the LDS writes ends with the first stage's loads,
  // which the first step waits for anyway at two stages).  The previous
  // tile's epilogue read these arrays before this tile's first barrier.
  float rwv = 0.f, rdv = 0.f;
  const bool rterm = MODE == DGRAD_UP && p.rdl != nullptr;
  if (rterm) {
    if (tid < BN) {
      const int col = w.nt * BN + tid;
      rwv = col < p.N ? bf2f(p.rw[(size_t)col * p.E + w.e]) : 0.f;
    }
    if (tid < BM) rdv = tid < w.rows ? p.rdl[w.row0 + tid] : 0.f;
  }
  if (0 < nk) issue(0, I0{});
  if (S > 2 && 1 < nk) issue(1, I1{});
  if (S > 3 && 2 < nk) issue(2, I2{});
  if constexpr (MODE == DGRAD_UP) {
    if (rterm) {
      if (tid < BN) rcol[tid] = rwv;
      if (tid < BM) rrow[tid] = rdv;
    }
  }
  // One K step on stage CUR, loading step kt+S-1 into stage NXT.  The wait
  // covers only this wave's loads of step kt (later steps stay in flight);
  // the barrier has no memory fence (a fence would drain every load).
  auto step = [&](int kt, auto cur, auto nxt, auto full) {
    const int after = min(S - 2, nk - 1 - kt);  // stages issued after kt so far
    // vmcnt(n): simm16 = vmcnt[3:0] | expcnt(7)<<4 | lgkmcnt(15)<<8 | vmcnt[5:4]<<14
    if (S >= 4 && after >= 2)
      __builtin_amdgcn_s_waitcnt(((2 * LPS) & 15) | (7 << 4) | (15 << 8) | (((2 * LPS) >> 4) << 14));
    else if (S >= 3 && after >= 1)
      __builtin_amdgcn_s_waitcnt((LPS & 15) | (7 << 4) | (15 << 8) | ((LPS >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (kt + S - 1 < nk) issue(kt + S - 1, nxt);
    compute(cur, full);
  };
  auto main_loop = [&](auto full) {
    int kt = 0;
    if constexpr (S == 2) {
      for (; kt + 1 < nk; kt += 2) {
        step(kt, I0{}, I1{}, full);
        step(kt + 1, I1{}, I0{}, full);
      }
      if (kt < nk) step(kt, I0{}, I1{}, full);
    } else if constexpr (S == 3) {
      for (; kt + 2 < nk; kt += 3) {
        step(kt, I0{}, I2{}, full);
        step(kt + 1, I1{}, I0{}, full);
        step(kt + 2, I2{}, I1{}, full);
      }
      if (kt < nk) step(kt, I0{}, I2{}, full);
      if (kt + 1 < nk) step(kt + 1, I1{}, I0{}, full);
    } else {
      for (; kt + 3 < nk; kt += 4) {
        step(kt, I0{}, I3{}, full);
        step(kt + 1, I1{}, I0{}, full);
        step(kt + 2, I2{}, I1{}, full);
        step(kt + 3, I3{}, I2{}, full);
      }
      if (kt < nk) step(kt, I0{}, I3{}, full);
      if (kt + 1 < nk) step(kt + 1, I1{}, I0{}, full);
      if (kt + 2 < nk) step(kt + 2, I2{}, I1{}, full);
    }
  };
  // full tiles run branch-free; a tile reaching into the strip runs the strip
  // MFMAs as well (its main subtiles are then all valid)
  const bool strip = TL::XR > 0 && w.rows > TL::BMAIN;
  if constexpr (TL::XR > 0) {
    if (strip)
      main_loop(std::integral_constant<int, 2>{});
    else if (nvsm == SM)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  } else {
    if (TR::kKRAGGED || nvsm == SM)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  }
  // all waves are done with the stage buffers before the block exits
  asm volatile("s_barrier" ::: "memory");
  // with the strip, the epilogue's lane-derived addresses are formed here,
  // not before the loop (where they would take the loop's registers)
  if constexpr (TL::XR > 0) asm volatile("" : "+v"(lane));

  if constexpr (MODE == DGRAD_UP) {
    if (p.rdl != nullptr) {
      // Router term of the input gradient, a rank-1 update of the fp32 tile:
      // acc[m][n] += dl(row m) * W_r[n][e], both factors staged in LDS at the
      // start of the tile.
      float dlv[SM];
#pragma unroll
      for (int sm = 0; sm < SM; ++sm) dlv[sm] = rrow[wm * TL::WM + sm * 32 + (lane & 31)];
      const int ncol4 = 4 * (lane >> 5);
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float wv = rcol[wn * 128 + sn * 32 + 8 * (r >> 2) + ncol4 + (r & 3)];
#pragma unroll
          for (int sm = 0; sm < SM; ++sm) acc[sm][sn][r] += dlv[sm] * wv;
        }
        // one column subtile at a time: its 16 W_r values are all that is live
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (TL::XR > 0) {
        if (strip) {
          const float dlx = rrow[TL::BMAIN + (lane & 31)];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            accx[0][0][r] += dlx * rcol[wn * 128 + wm * 32 + 8 * (r >> 2) + ncol4 + (r & 3)];
        }
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  EpiArgs ea{p.c0, p.c1, p.c2, p.ldc, p.c_gstride, p.aux0, p.aux1, p.N, p.M};
  // The strip's 32x32 tile of this wave (rows BMAIN.., columns wn*128 +
  // wm*32.. of the block tile).  The down dgrad stores it first, straight
  // from the accumulators (its SwiGLU backward needs them in fp32); the
  // gate/up dgrad rounds it to bf16 here and stores it after the main
  // epilogue, so only eight registers stay live through that.
  [[maybe_unused]] uint32_t xpk[8];
  if constexpr (TL::XR > 0) {
    if (strip) {
      if constexpr (MODE == DGRAD_DOWN) {
        Work ws = w;
        ws.row0 = w.row0 + TL::BMAIN;
        ws.rows = w.rows - TL::BMAIN;
        store_tile_direct<MODE, BM, 1, false, 1, 32>(accx, ea, ws, lane, 0, wn * 4 + wm);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xpk[i] = pack2bf(accx[0][0][2 * i], accx[0][0][2 * i + 1]);
      }
    }
  }
  if constexpr (TR::kKRAGGED) {
    if (p.part) {
      store_partial_f32<MODE, BM, SM>(acc, ea, w, lane, wm, wn);
      continue;
    }
  }
  if constexpr (epi_staged<MODE, NW>(TL::STAGE, S)) {
    constexpr int CH = epi_chunk<MODE, NW>(TL::STAGE, S);
    constexpr int NCS = epi_ncs<MODE, NW>(TL::STAGE, S);
    constexpr int REG = epi_region_bytes<MODE>(CH, NCS);
    constexpr int PER = TL::STAGE / REG;
    static_assert(S * PER >= NW, "epilogue staging regions do not fit the stage buffers");
    const int sel = wave / PER;
    LDS_AS unsigned char* wbuf =
        (sel == 0 ? (LDS_AS unsigned char*)lds0 : sel == 1 ? (LDS_AS unsigned char*)lds1
         : sel == 2 ? (LDS_AS unsigned char*)lds2 : (LDS_AS unsigned char*)lds3) + (wave % PER) * REG;
    store_tile<MODE, BM, SM, false, CH, NCS, (TL::XR > 0)>(acc, ea, w, lane, wm, wn, wbuf);
  } else {
    store_tile_direct<MODE, BM, SM, false>(acc, ea, w, lane, wm, wn);
  }
  if constexpr (TL::XR > 0 && MODE != DGRAD_DOWN) {
    // lane holds row BMAIN + (lane & 31), columns 8*g + 4*(lane >> 5) + 0..3
    if (strip && (lane & 31) < w.rows - TL::BMAIN) {
      const size_t crow = (size_t)(w.row0 + TL::BMAIN + (lane & 31));
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = w.nt * BN + wn * 128 + wm * 32 + 8 * g4 + 4 * (lane >> 5);
        if (col < p.N)
          *reinterpret_cast<uint2*>((bf16_t*)p.c0 + crow * p.ldc + col) =
              make_uint2(xpk[2 * g4], xpk[2 * g4 + 1]);
      }
    }
  }
  }  // tiles of this block
#endif
}

// Launch over `blocks` (the tile bound of the launch, rounded up to whole
// XCD rounds); blocks past the real tile count exit.
template <int MODE, int BM, int S, int BK, int OCC = 1, int NW = 4, bool NF = false>
hipError_t launch(const Params& p, int blocks, hipStream_t s) {
  blocks = (blocks + 7) / 8 * 8;
  grouped_gemm_kernel<MODE, BM, S, BK, OCC, NW, NF><<<blocks, 64 * NW, 0, s>>>(p);
  return hipGetLastError();
}

// Tile configurations: rows per tile, pipeline stages, K step, blocks per
// CU, waves per block.  Two resident blocks per CU (128x256 tiles, 32-deep K
// steps in three stages, 72 KiB of LDS, at most 256 registers per wave) let
// one block's prologue, barriers and output stores overlap the other block's
// MFMAs on the same SIMDs; the forward GEMMs and the wgrads run so.  The two
// dgrads instead run one 256x256 block per CU with eight waves (64x128 wave
// tiles, two waves per SIMD) and 64-deep K steps in two 64 KiB stages: a
// third less L2->LDS traffic per FLOP and half the barriers, which outweighs
// the lost overlap there.  Their tiles carry the 32-row strip (288 rows, two
// 68 KiB stages): with a few hundred routed rows per expert, an expert just
// past 512 rows then takes two row tiles instead of two plus a nearly empty
// third that would still stream the whole weight tile (uniform top-4 over 128
// experts, 454-564 rows each: down dgrad 0.45 -> 0.41 ms, gate/up dgrad
// 0.69 -> 0.65 ms; on Zipf-skewed counts both run about 6 % slower, on 8192
// rows per expert the down dgrad is 10 % faster and the gate/up dgrad 7 %
// slower).  In the forward GEMMs, whose epilogues are heavier,
// 256-row tiles lose: at a few hundred rows per expert an expert's last
// 256-row tile is often nearly empty yet loads a full weight tile (measured
// per mode on routed counts).  (The down dgrad's epilogue, which also streams
// the saved g and u, stages its columns in two 64-column passes of 32 rows
// to bound its registers.)
#ifndef GEMM_M_CFG
#define GEMM_M_CFG 128, 3, 32, 2   // forward gate/up and down
#endif
#ifndef GEMM_UP_CFG
#define GEMM_UP_CFG GEMM_M_CFG     // forward gate/up
#endif
#ifndef GEMM_DN_CFG
#define GEMM_DN_CFG GEMM_M_CFG     // forward down
#endif
#ifndef GEMM_DU_CFG
#define GEMM_DU_CFG 288, 2, 64, 1, 8  // gate/up dgrad
#endif
#ifndef GEMM_DD_CFG
#define GEMM_DD_CFG 288, 2, 64, 1, 8  // down dgrad
#endif
#ifndef GEMM_W_CFG
#define GEMM_W_CFG 128, 3, 32, 2   // both wgrads
#endif
#ifndef GEMM_WU_CFG
#define GEMM_WU_CFG GEMM_W_CFG     // gate/up wgrad
#endif
#ifndef GEMM_WD_CFG
#define GEMM_WD_CFG GEMM_W_CFG     // down wgrad
#endif
// rows, stages, K step, blocks per CU, waves per block (NW/2 down, 2 across)
template <int BM_, int S_, int BK_, int OCC_, int NW_ = 4>
struct Cfg {
  static constexpr int BM = BM_, S = S_, BK = BK_, OCC = OCC_, NW = NW_;
};
using CfgUP = Cfg<GEMM_UP_CFG>;
using CfgDN = Cfg<GEMM_DN_CFG>;
using CfgDU = Cfg<GEMM_DU_CFG>;
using CfgDD = Cfg<GEMM_DD_CFG>;
using CfgWU = Cfg<GEMM_WU_CFG>;
using CfgWD = Cfg<GEMM_WD_CFG>;

// Upper bound of sum_e ceil(n_e / BM) over any split of R rows into E groups.
int mtile_bound(int R, int E, int BM) { return R / BM + E; }

}  // namespace

// ---------------------------------------------------------------- host API
using namespace moe_host;

// Launch of a row-ragged mode with its tile configuration; the grid is the
// bound on sum_e ceil(n_e / BM) tiles, found on the device.
template <int MODE>
static hipError_t launch_mragged(Params& p, int R, hipStream_t s) {
  using C = std::conditional_t<
      MODE == DGRAD_DOWN, CfgDD,
      std::conditional_t<MODE == DGRAD_UP, CfgDU, std::conditional_t<MODE == FWD_UP, CfgUP, CfgDN>>>;
  // (+8 plan blocks at the end of the grid when the down dgrad plans the
  // weight gradients' ranges; the tile count is rounded to a multiple of 8)
  const int tiles = (mtile_bound(R, p.E, C::BM) * p.ntiles + 7) / 8 * 8;
  const int blocks = tiles + (p.xr_out0 != nullptr ? 8 : 0);
  // Order of an expert's tiles within its XCD range, measured per mode on
  // routed counts: the dgrads walk each row tile across its n-tiles
  // (uniform top-4 over 128 experts: down dgrad 0.417 -> 0.399 ms, gate/up
  // dgrad 0.672 -> 0.649; 8192 rows per expert and Zipf-skewed counts gain
  // 5-10 %).  The forward GEMMs do so only when the average expert holds at
  // least as many row tiles as column tiles (R / E >= BM * ntiles): with
  // fewer, the blocks that run at once share each weight tile better in
  // n-major order (uniform top-4 over 128 experts, 4-5 row tiles per
  // expert: gate/up 0.664 ms n-major against 0.70 m-major), with more they
  // share the row tiles (8192 rows per expert: gate/up 0.66 -> 0.60 ms,
  // down 0.334 -> 0.312).
  if constexpr (MODE == DGRAD_DOWN || MODE == DGRAD_UP) {
    return launch<MODE, C::BM, C::S, C::BK, C::OCC, C::NW, true>(p, blocks, s);
  } else {
    if (p.E > 0 && (long long)R >= (long long)p.E * C::BM * p.ntiles)
      return launch<MODE, C::BM, C::S, C::BK, C::OCC, C::NW, true>(p, blocks, s);
    return launch<MODE, C::BM, C::S, C::BK, C::OCC, C::NW, false>(p, blocks, s);
  }
}

moe_status moe_internal_router_logits_mfma(moe_ctx* ctx, const void* x, const void* wr, int T_,
                                           int d, int E, float* logits) {
  if (d % 64 != 0)
    return fail(ctx, MOE_ERR_UNSUPPORTED, "moe_router_logits: MFMA path needs d %% 64 == 0");
  Params p{};
  p.a0 = (const bf16_t*)x;
  p.lda = d;
  p.b0 = (const bf16_t*)wr;
  p.ldb = E;
  p.c0 = logits;
  p.ldc = E;
  p.M = T_;
  p.N = E;
  p.K = d;
  p.kseg = d;
  p.ntiles = (E + BN - 1) / BN;
  p.E = 1;
  // 64-row tiles: T/64 blocks fill the chip for the token counts the layer
  // runs at (the scores GEMM is bound by reading x once)
  constexpr int kRouterBM = 64;
  const int blocks = ((T_ + kRouterBM - 1) / kRouterBM) * p.ntiles;
  hipError_t e = launch<ROUTER, kRouterBM, 4, 32, 1>(p, blocks, ctx->stream);
  if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "router GEMM: %s", hipGetErrorString(e));
  return MOE_OK;
}

// The router's share of a dense logit gradient on the matrix cores (bf16
// operands, fp32 sums; dlb is the gradient rounded to bf16, wrt = W_r^T
// [E,d]):
//   dx[T,d] += dlb[T,E] wrt[E,d]: the one-group score GEMM (MODE 6) whose
//     epilogue adds each fp32 tile into dx and rounds once;
//   part[g][d][E] = x_g^T dlb_g for the token chunks g of voff (nz chunks):
//     the K-ragged down-wgrad GEMM (MODE 5) over the chunks as groups,
//     storing exact fp32 partials that the caller sums in chunk order.
// Needs d % 64 == 0 and E % 64 == 0.
moe_status moe_internal_router_dense_mfma(moe_ctx* ctx, const bf16_t* x, const bf16_t* dlb,
                                          const bf16_t* wrt, const int32_t* voff, int nz, int T_,
                                          int d, int E, bf16_t* dx, float* part) {
  hipError_t e;
  {
    Params p{};
    p.a0 = dlb;
    p.lda = E;
    p.b0 = wrt;
    p.ldb = d;
    p.c0 = dx;
    p.aux0 = dx;
    p.ldc = d;
    p.M = T_;
    p.N = d;
    p.K = E;
    p.kseg = E;
    p.ntiles = (d + BN - 1) / BN;
    p.E = 1;
    constexpr int kBM = 64;
    const int blocks = ((T_ + kBM - 1) / kBM) * p.ntiles;
    e = launch<ROUTER, kBM, 4, 32, 1>(p, blocks, ctx->stream);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "router dense dx GEMM: %s", hipGetErrorString(e));
  }
  {
    Params p{};
    p.a0 = x;
    p.lda = d;
    p.b0 = dlb;
    p.ldb = E;
    p.c0 = part;
    p.ldc = E;
    p.c_gstride = (long long)d * E;
    p.offsets = voff;
    p.E = nz;
    p.M = d;
    p.N = E;
    p.ntiles = (E + BN - 1) / BN;
    p.mtiles = (d + CfgWD::BM - 1) / CfgWD::BM;
    p.part = 1;
    e = launch<WGRAD_DOWN, CfgWD::BM, CfgWD::S, CfgWD::BK, CfgWD::OCC, CfgWD::NW>(p, nz * p.ntiles * p.mtiles,
                                                                              ctx->stream);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "router dense dW GEMM: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

// fp32 path (gemm_f32.hip)
moe_status moe_internal_ffn_fwd_f32(moe_ctx* ctx, const float* xp, const float* wg,
                                    const float* wu, const float* wd, const int32_t* offsets,
                                    int E, int R, int d, int F, float* g, float* u, float* h,
                                    float* yp);
moe_status moe_internal_ffn_bwd_f32(moe_ctx* ctx, const float* xp, const float* wg,
                                    const float* wu, const float* wd, const int32_t* offsets,
                                    const float* g, const float* u, const float* h,
                                    const float* dyp, int E, int R, int d, int F, float* dg,
                                    float* du, float* dxp, float* dwg, float* dwu, float* dwd);

// MXFP8 path (gemm_mx.hip)
size_t moe_internal_mx_fwd_bytes(int E, int R, int d, int F);
size_t moe_internal_mx_bwd_bytes(int E, int R, int d, int F);
moe_status moe_internal_ffn_fwd_mx(moe_ctx* ctx, const bf16_t* xp, const uint8_t* xq_in,
                                   const uint8_t* xs_in, const bf16_t* wg, const bf16_t* wu,
                                   const bf16_t* wd, const MxWeights* pw, const int32_t* offsets,
                                   int E, int R, int d, int F, bf16_t* g, bf16_t* u, bf16_t* h,
                                   bf16_t* yp);
moe_status moe_internal_ffn_bwd_mx(moe_ctx* ctx, const bf16_t* xp, const bf16_t* wg,
                                   const bf16_t* wu, const bf16_t* wd, const MxWeights* pw,
                                   const int32_t* offsets, const bf16_t* g, const bf16_t* u,
                                   const bf16_t* h, const bf16_t* dyp, int E, int R, int d, int F,
                                   bf16_t* dg, bf16_t* du, bf16_t* dxp, bf16_t* dwg, bf16_t* dwu,
                                   bf16_t* dwd, bool wgrad_bf16);
size_t moe_internal_mx_pack_layout(int E, int d, int F, uint8_t* base, MxWeights* w);
moe_status moe_internal_mx_quantize_weights(moe_ctx* ctx, const bf16_t* wg, const bf16_t* wu,
                                            const bf16_t* wd, int E, int d, int F, uint8_t* pack);

// ---------------------------------------------------------------- split-K
// A weight-gradient launch has E * mtiles * ntiles output tiles.  When that
// leaves block slots idle (fewer than two tiles per CU) and the groups are
// long (a shared expert: one group of every token), each group's K range is
// cut into S segments of whole 32-row steps, run as S virtual groups that
// store exact fp32 partial products, then summed in segment order and
// rounded once.  The choice depends only on the shapes and the chip.
static int wgrad_splits(int E, int R, int tiles) {
  const int slots = 2 * moe_host::device_cus();
  if (E <= 0 || tiles <= 0 || tiles >= slots) return 1;
  const long long avg = (long long)R / E;
  if (avg < 1024) return 1;
  long long s = (slots + tiles - 1) / tiles;
  s = std::min<long long>(s, 8);
  s = std::min<long long>(s, avg / 256);
  return (int)std::max<long long>(s, 1);
}
static int wgrad_up_tiles(int E, int d, int F) { return E * ((d + CfgWU::BM - 1) / CfgWU::BM) * ((F + 127) / 128); }
static int wgrad_down_tiles(int E, int d, int F) { return E * ((F + CfgWD::BM - 1) / CfgWD::BM) * ((d + BN - 1) / BN); }
// Workspace of the split weight gradients: the partials of the larger one
// (gate/up: two [E*S, d, F] fp32 arrays) followed by the virtual offsets.
// The bf16 backward's workspace: the XCD range tables of the two weight
// gradients (kPlanBytes), then the split-K partials and virtual offsets.
constexpr size_t kPlanBytes = 256;
static size_t wgrad_split_bytes(int E, int R, int d, int F, size_t* part_bytes) {
  const int su = wgrad_splits(E, R, wgrad_up_tiles(E, d, F));
  const int sd = wgrad_splits(E, R, wgrad_down_tiles(E, d, F));
  if (su == 1 && sd == 1) {
    *part_bytes = 0;
    return 0;
  }
  const size_t up = su > 1 ? 2 * (size_t)E * su * d * F * 4 : 0;
  const size_t dn = sd > 1 ? (size_t)E * sd * F * d * 4 : 0;
  *part_bytes = ((up > dn ? up : dn) + 255) & ~(size_t)255;
  return *part_bytes + (((size_t)E * 8 + 1) * 4 + 255) / 256 * 256;
}

// Per-XCD tile ranges of a split-K weight gradient over its virtual groups:
// one wave per XCD, xr[2x], xr[2x+1] = [first, end) of XCD x.
__global__ void __launch_bounds__(512) xcd_plan_kernel(const int32_t* __restrict__ off, int E,
                                                       int per_e, int32_t* __restrict__ xr) {
  const int x = threadIdx.x >> 6;
  int first, end;
  kragged_xcd_range<kWgradBK>(off, E, per_e, x, first, end);
  if ((threadIdx.x & 63) == 0) {
    xr[2 * x] = first;
    xr[2 * x + 1] = end;
  }
}

__global__ void split_offsets_kernel(const int32_t* __restrict__ off, int E, int S,
                                     int32_t* __restrict__ voff) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i > E * S) return;
  if (i == E * S) {
    voff[i] = off[E];
    return;
  }
  const int e = i / S, sgm = i % S;
  const int lo = off[e], len = off[e + 1] - lo;
  const int seg = ((len + S - 1) / S + 31) / 32 * 32;
  voff[i] = lo + min(len, sgm * seg);
}

// out[e][j] = bf16(sum_s part[e*S + s][j]) in segment order; n4 = float4s per group.
__global__ void split_reduce_kernel(const float4* __restrict__ part, int S, long long n4,
                                    long long total4, uint2* __restrict__ out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total4) return;
  const long long e = i / n4, j = i - e * n4;
  float4 acc = part[(e * S) * n4 + j];
  for (int sg = 1; sg < S; ++sg) {
    const float4 v = part[(e * S + sg) * n4 + j];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  out[i] = make_uint2(pack2bf(acc.x, acc.y), pack2bf(acc.z, acc.w));
}

static hipError_t split_reduce(const float* part, int E, int S, size_t n, bf16_t* out, hipStream_t s) {
  const long long n4 = (long long)(n / 4), total4 = (long long)E * n4;
  split_reduce_kernel<<<(unsigned)((total4 + 255) / 256), 256, 0, s>>>((const float4*)part, S, n4,
                                                                       total4, (uint2*)out);
  return hipGetLastError();
}

// The two bf16 weight gradients (K-ragged over each expert's rows).  plan_*:
// the XCD range table of the launch (planned: filled from the routed counts
// before this launch, else equal tile counts per XCD); split_part and
// split_voff: the split-K workspace (wgrad_split_bytes).
static moe_status run_wgrad_down(moe_ctx* ctx, const void* h, const void* dyp, const int32_t* offsets,
                                 int E, int R, int d, int F, void* dw_down, int32_t* plan_dn, bool planned,
                                 float* split_part, int32_t* split_voff) {
  const int dn_per_e = ((d + BN - 1) / BN) * ((F + CfgWD::BM - 1) / CfgWD::BM);
  hipError_t e;
  {
    // down wgrad: dWd[e] = h_e^T dyp_e (M = F, N = d, K = rows of e)
    Params p{};
    p.a0 = (const bf16_t*)h;
    p.lda = F;
    p.b0 = (const bf16_t*)dyp;
    p.ldb = d;
    p.c0 = dw_down;
    p.ldc = d;
    p.c_gstride = (long long)F * d;
    p.offsets = offsets;
    p.E = E;
    p.M = F;
    p.N = d;
    p.ntiles = (d + BN - 1) / BN;
    p.mtiles = (F + CfgWD::BM - 1) / CfgWD::BM;
    {
      moe_prof_scope ps(ctx, MOE_K_GEMM_WGRAD_DOWN);
      const int S = wgrad_splits(E, R, E * p.ntiles * p.mtiles);
      if (S == 1) {
        p.xr = planned ? plan_dn : nullptr;
        e = launch<WGRAD_DOWN, CfgWD::BM, CfgWD::S, CfgWD::BK, CfgWD::OCC, CfgWD::NW>(p, E * p.ntiles * p.mtiles,
                                                                      ctx->stream);
      } else {
        split_offsets_kernel<<<(E * S + 256) / 256, 256, 0, ctx->stream>>>(offsets, E, S, split_voff);
        xcd_plan_kernel<<<1, 512, 0, ctx->stream>>>(split_voff, E * S, dn_per_e, plan_dn);
        Params q = p;
        q.offsets = split_voff;
        q.E = E * S;
        q.xr = plan_dn;
        q.c0 = split_part;
        q.part = 1;
        e = launch<WGRAD_DOWN, CfgWD::BM, CfgWD::S, CfgWD::BK, CfgWD::OCC, CfgWD::NW>(q, q.E * q.ntiles * q.mtiles,
                                                                      ctx->stream);
        if (e == hipSuccess) e = split_reduce(split_part, E, S, (size_t)F * d, (bf16_t*)dw_down, ctx->stream);
      }
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "down wgrad: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

static moe_status run_wgrad_up(moe_ctx* ctx, const void* xp, const void* dg, const void* du,
                               const int32_t* offsets, int E, int R, int d, int F, void* dw_gate, void* dw_up,
                               int32_t* plan_up, bool planned, float* split_part, int32_t* split_voff) {
  const int up_per_e = ((F + 127) / 128) * ((d + CfgWU::BM - 1) / CfgWU::BM);
  hipError_t e;
  {
    // gate/up wgrad: dWg[e] = xp_e^T dg_e, dWu[e] = xp_e^T du_e (M = d, N = F each)
    Params p{};
    p.a0 = (const bf16_t*)xp;
    p.lda = d;
    p.b0 = (const bf16_t*)dg;
    p.b1 = (const bf16_t*)du;
    p.ldb = F;
    p.c0 = dw_gate;
    p.c1 = dw_up;
    p.ldc = F;
    p.c_gstride = (long long)d * F;
    p.offsets = offsets;
    p.E = E;
    p.M = d;
    p.N = F;
    p.ntiles = (F + 127) / 128;
    p.mtiles = (d + CfgWU::BM - 1) / CfgWU::BM;
    {
      moe_prof_scope ps(ctx, MOE_K_GEMM_WGRAD_UP);
      const int S = wgrad_splits(E, R, E * p.ntiles * p.mtiles);
      if (S == 1) {
        p.xr = planned ? plan_up : nullptr;
        e = launch<WGRAD_UP, CfgWU::BM, CfgWU::S, CfgWU::BK, CfgWU::OCC, CfgWU::NW>(p, E * p.ntiles * p.mtiles,
                                                                    ctx->stream);
      } else {
        split_offsets_kernel<<<(E * S + 256) / 256, 256, 0, ctx->stream>>>(offsets, E, S, split_voff);
        xcd_plan_kernel<<<1, 512, 0, ctx->stream>>>(split_voff, E * S, up_per_e, plan_up);
        Params q = p;
        q.offsets = split_voff;
        q.E = E * S;
        q.xr = plan_up;
        q.c0 = split_part;
        q.c1 = split_part + (size_t)E * S * d * F;
        q.part = 1;
        e = launch<WGRAD_UP, CfgWU::BM, CfgWU::S, CfgWU::BK, CfgWU::OCC, CfgWU::NW>(q, q.E * q.ntiles * q.mtiles,
                                                                    ctx->stream);
        if (e == hipSuccess) e = split_reduce(split_part, E, S, (size_t)d * F, (bf16_t*)dw_gate, ctx->stream);
        if (e == hipSuccess)
          e = split_reduce(split_part + (size_t)E * S * d * F, E, S, (size_t)d * F, (bf16_t*)dw_up,
                           ctx->stream);
      }
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "gate/up wgrad: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

size_t moe_internal_wgrads_bf16_bytes(int E, int R, int d, int F) {
  size_t part = 0;
  return kPlanBytes + wgrad_split_bytes(E, R, d, F, &part);
}

// Both bf16 weight gradients after data gradients computed elsewhere (the
// MXFP8 backward with bf16 weight gradients): the XCD range tables come from
// the routed counts (one small launch), then the two launches as in the bf16
// backward.  ws: moe_internal_wgrads_bf16_bytes(E, R, d, F) bytes.
moe_status moe_internal_wgrads_bf16(moe_ctx* ctx, const bf16_t* xp, const int32_t* offsets,
                                    const bf16_t* dg, const bf16_t* du, const bf16_t* h,
                                    const bf16_t* dyp, int E, int R, int d, int F, bf16_t* dwg,
                                    bf16_t* dwu, bf16_t* dwd, void* ws) {
  size_t part_bytes = 0;
  wgrad_split_bytes(E, R, d, F, &part_bytes);
  int32_t* plan_dn = (int32_t*)ws;
  int32_t* plan_up = plan_dn + 16;
  float* split_part = (float*)((char*)ws + kPlanBytes);
  int32_t* split_voff = (int32_t*)((char*)ws + kPlanBytes + part_bytes);
  const bool planned = R > 0;
  if (planned) {
    static_assert(CfgWD::BK == kWgradBK && CfgWU::BK == kWgradBK, "weight-gradient plans use kWgradBK");
    const int dn_per_e = ((d + BN - 1) / BN) * ((F + CfgWD::BM - 1) / CfgWD::BM);
    const int up_per_e = ((F + 127) / 128) * ((d + CfgWU::BM - 1) / CfgWU::BM);
    xcd_plan_kernel<<<1, 512, 0, ctx->stream>>>(offsets, E, dn_per_e, plan_dn);
    xcd_plan_kernel<<<1, 512, 0, ctx->stream>>>(offsets, E, up_per_e, plan_up);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "weight-gradient plan: %s", hipGetErrorString(e));
  }
  moe_status st = run_wgrad_down(ctx, h, dyp, offsets, E, R, d, F, dwd, plan_dn, planned, split_part, split_voff);
  if (st != MOE_OK) return st;
  return run_wgrad_up(ctx, xp, dg, du, offsets, E, R, d, F, dwg, dwu, plan_up, planned, split_part, split_voff);
}

static moe_status ffn_validate(moe_ctx* ctx, int E, int R, int d, int F, moe_dtype dtype,
                               const char* what) {
  MOE_REQUIRE(ctx, dtype == MOE_F32 || dtype == MOE_BF16 || dtype == MOE_MXFP8,
              "%s: unsupported dtype %d", what, (int)dtype);
  MOE_REQUIRE(ctx, E >= 1 && E <= 1024 && R >= 0 && d >= 8 && F >= 8 && d % 8 == 0 && F % 8 == 0,
              "%s: bad shape E=%d R=%d d=%d F=%d", what, E, R, d, F);
  if (dtype == MOE_BF16 && (d % 64 != 0 || F % 64 != 0))
    return fail(ctx, MOE_ERR_UNSUPPORTED, "%s: bf16 path needs d and F multiples of 64", what);
  if (dtype == MOE_MXFP8 && (d % 128 != 0 || F % 128 != 0))
    return fail(ctx, MOE_ERR_UNSUPPORTED, "%s: MXFP8 path needs d and F multiples of 128", what);
  MOE_REQUIRE(ctx, (int64_t)R * (d > F ? d : F) * 2 < ((int64_t)1 << 31),
              "%s: R * max(d, F) too large for 32-bit buffer offsets", what);
  return MOE_OK;
}

extern "C" {

moe_status moe_mx_workspace_size(moe_ctx* ctx, int E, int R, int d, int F, size_t* bytes) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, bytes != nullptr, "bytes is null");
  moe_status st = ffn_validate(ctx, E, R, d, F, MOE_MXFP8, "moe_mx_workspace_size");
  if (st != MOE_OK) return st;
  // (the backward with bf16 weight gradients keeps their workspace after the
  // MXFP8 layout)
  const size_t a = moe_internal_mx_fwd_bytes(E, R, d, F),
               b = moe_internal_mx_bwd_bytes(E, R, d, F) + moe_internal_wgrads_bf16_bytes(E, R, d, F);
  *bytes = a > b ? a : b;
  return MOE_OK;
}

moe_status moe_ffn_bwd_workspace_size(moe_ctx* ctx, int E, int R, int d, int F, moe_dtype dtype,
                                      size_t* bytes) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, bytes != nullptr, "bytes is null");
  moe_status st = ffn_validate(ctx, E, R, d, F, dtype, "moe_ffn_bwd_workspace_size");
  if (st != MOE_OK) return st;
  size_t part = 0;
  if (dtype == MOE_MXFP8)
    *bytes = moe_internal_mx_bwd_bytes(E, R, d, F);
  else if (dtype == MOE_BF16)
    *bytes = kPlanBytes + wgrad_split_bytes(E, R, d, F, &part);
  else
    *bytes = 0;
  return MOE_OK;
}

moe_status moe_grouped_ffn_fwd(moe_ctx* ctx, const void* xp, const void* w_gate,
                               const void* w_up, const void* w_down, const int32_t* offsets,
                               int E, int R, int d, int F, moe_dtype dtype, void* g, void* u,
                               void* h, void* yp) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, R, d, F, dtype, "moe_grouped_ffn_fwd");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp, R == 0);
  MOE_REQUIRE_PTR(ctx, w_gate);
  MOE_REQUIRE_PTR(ctx, w_up);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, g, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, u, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, h, R == 0);
  // w_down and yp both NULL: the gate/up GEMM alone (recompute of g, u, h)
  const bool up_only = w_down == nullptr && yp == nullptr;
  if (!up_only) {
    MOE_REQUIRE_PTR(ctx, w_down);
    MOE_REQUIRE_PTR_OR_EMPTY(ctx, yp, R == 0);
  }
  {
    const size_t es = dtype == MOE_F32 ? 4 : 2, rf = (size_t)R * F * es;
    MOE_REQUIRE_DISJOINT(ctx, "moe_grouped_ffn_fwd", {g, rf, "g"}, {u, rf, "u"}, {h, rf, "h"},
                         {yp, (size_t)R * d * es, "yp"});
  }
  if (R == 0) return MOE_OK;
  if (dtype == MOE_MXFP8)
    return moe_internal_ffn_fwd_mx(ctx, (const bf16_t*)xp, nullptr, nullptr, (const bf16_t*)w_gate,
                                   (const bf16_t*)w_up, (const bf16_t*)w_down, nullptr, offsets, E, R, d, F,
                                   (bf16_t*)g, (bf16_t*)u, (bf16_t*)h, (bf16_t*)yp);
  if (dtype == MOE_F32)
    return moe_internal_ffn_fwd_f32(ctx, (const float*)xp, (const float*)w_gate,
                                    (const float*)w_up, (const float*)w_down, offsets, E, R, d, F,
                                    (float*)g, (float*)u, (float*)h, (float*)yp);
  hipError_t e;
  {
    Params p{};
    p.a0 = (const bf16_t*)xp;
    p.lda = d;
    p.b0 = (const bf16_t*)w_gate;
    p.b1 = (const bf16_t*)w_up;
    p.ldb = F;
    p.b_gstride = (long long)d * F;
    p.c0 = g;
    p.c1 = u;
    p.c2 = h;
    p.ldc = F;
    p.offsets = offsets;
    p.E = E;
    p.N = F;
    p.K = d;
    p.kseg = d;
    p.ntiles = (F + 127) / 128;
    {
      moe_prof_scope ps(ctx, MOE_K_GEMM_UP);
      e = launch_mragged<FWD_UP>(p, R, ctx->stream);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "gate/up GEMM: %s", hipGetErrorString(e));
  }
  if (up_only) return MOE_OK;
  {
    Params p{};
    p.a0 = (const bf16_t*)h;
    p.lda = F;
    p.b0 = (const bf16_t*)w_down;
    p.ldb = d;
    p.b_gstride = (long long)F * d;
    p.c0 = yp;
    p.ldc = d;
    p.offsets = offsets;
    p.E = E;
    p.N = d;
    p.K = F;
    p.kseg = F;
    p.ntiles = (d + BN - 1) / BN;
    {
      moe_prof_scope ps(ctx, MOE_K_GEMM_DOWN);
      e = launch_mragged<FWD_DOWN>(p, R, ctx->stream);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "down GEMM: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

moe_status moe_grouped_ffn_fwd_mxq(moe_ctx* ctx, const uint8_t* xp_codes, const uint8_t* xp_scales,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const int32_t* offsets, int E, int R, int d, int F, void* g,
                                   void* u, void* h, void* yp) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, R, d, F, MOE_MXFP8, "moe_grouped_ffn_fwd_mxq");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp_codes, R == 0);
  MOE_REQUIRE(ctx, R == 0 || xp_scales != nullptr, "moe_grouped_ffn_fwd_mxq: xp_scales is null");
  MOE_REQUIRE_PTR(ctx, w_gate);
  MOE_REQUIRE_PTR(ctx, w_up);
  MOE_REQUIRE_PTR(ctx, w_down);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, g, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, u, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, h, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, yp, R == 0);
  {
    const size_t rf = (size_t)R * F * 2;
    MOE_REQUIRE_DISJOINT(ctx, "moe_grouped_ffn_fwd_mxq", {g, rf, "g"}, {u, rf, "u"}, {h, rf, "h"},
                         {yp, (size_t)R * d * 2, "yp"});
  }
  if (R == 0) return MOE_OK;
  return moe_internal_ffn_fwd_mx(ctx, nullptr, xp_codes, xp_scales, (const bf16_t*)w_gate,
                                 (const bf16_t*)w_up, (const bf16_t*)w_down, nullptr, offsets, E, R, d, F,
                                 (bf16_t*)g, (bf16_t*)u, (bf16_t*)h, (bf16_t*)yp);
}

moe_status moe_mx_weight_pack_size(moe_ctx* ctx, int E, int d, int F, size_t* bytes) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, bytes != nullptr, "bytes is null");
  moe_status st = ffn_validate(ctx, E, 0, d, F, MOE_MXFP8, "moe_mx_weight_pack_size");
  if (st != MOE_OK) return st;
  *bytes = moe_internal_mx_pack_layout(E, d, F, nullptr, nullptr);
  return MOE_OK;
}

// The pack a call was given, checked against its shape.
static moe_status pack_regions(moe_ctx* ctx, const void* pack, size_t pack_bytes, int E, int d, int F,
                               const char* what, MxWeights* w) {
  MOE_REQUIRE(ctx, pack != nullptr && (reinterpret_cast<uintptr_t>(pack) & 255u) == 0,
              "%s: pack null or not 256-byte aligned", what);
  const size_t need = moe_internal_mx_pack_layout(E, d, F, nullptr, nullptr);
  MOE_REQUIRE(ctx, pack_bytes >= need, "%s: pack of %zu bytes < %zu for E=%d d=%d F=%d", what,
              pack_bytes, need, E, d, F);
  moe_internal_mx_pack_layout(E, d, F, (uint8_t*)pack, w);
  return MOE_OK;
}

moe_status moe_mx_quantize_weights(moe_ctx* ctx, const void* w_gate, const void* w_up,
                                   const void* w_down, int E, int d, int F, void* pack,
                                   size_t pack_bytes) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, 0, d, F, MOE_MXFP8, "moe_mx_quantize_weights");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(ctx, w_gate);
  MOE_REQUIRE_PTR(ctx, w_up);
  MOE_REQUIRE_PTR(ctx, w_down);
  MxWeights w;
  st = pack_regions(ctx, pack, pack_bytes, E, d, F, "moe_mx_quantize_weights", &w);
  if (st != MOE_OK) return st;
  return moe_internal_mx_quantize_weights(ctx, (const bf16_t*)w_gate, (const bf16_t*)w_up,
                                          (const bf16_t*)w_down, E, d, F, (uint8_t*)pack);
}

moe_status moe_grouped_ffn_fwd_mxp(moe_ctx* ctx, const void* xp, const uint8_t* xp_codes,
                                   const uint8_t* xp_scales, const void* pack, size_t pack_bytes,
                                   const int32_t* offsets, int E, int R, int d, int F, void* g,
                                   void* u, void* h, void* yp) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, R, d, F, MOE_MXFP8, "moe_grouped_ffn_fwd_mxp");
  if (st != MOE_OK) return st;
  MOE_REQUIRE(ctx, R == 0 || (xp != nullptr) != (xp_codes != nullptr),
              "moe_grouped_ffn_fwd_mxp: give exactly one of xp and xp_codes");
  if (xp_codes) {
    MOE_REQUIRE_PTR(ctx, xp_codes);
    MOE_REQUIRE(ctx, xp_scales != nullptr, "moe_grouped_ffn_fwd_mxp: xp_scales is null");
  } else {
    MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp, R == 0);
  }
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, g, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, u, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, h, R == 0);
  if (yp) MOE_REQUIRE_PTR(ctx, yp);
  {
    const size_t rf = (size_t)R * F * 2;
    MOE_REQUIRE_DISJOINT(ctx, "moe_grouped_ffn_fwd_mxp", {g, rf, "g"}, {u, rf, "u"}, {h, rf, "h"},
                         {yp, (size_t)R * d * 2, "yp"});
  }
  MxWeights w;
  st = pack_regions(ctx, pack, pack_bytes, E, d, F, "moe_grouped_ffn_fwd_mxp", &w);
  if (st != MOE_OK) return st;
  if (R == 0) return MOE_OK;
  return moe_internal_ffn_fwd_mx(ctx, (const bf16_t*)xp, xp_codes, xp_scales, nullptr, nullptr, nullptr,
                                 &w, offsets, E, R, d, F, (bf16_t*)g, (bf16_t*)u, (bf16_t*)h,
                                 (bf16_t*)yp);
}

moe_status moe_grouped_ffn_bwd_mxp(moe_ctx* ctx, const void* xp, const void* pack,
                                   size_t pack_bytes, const int32_t* offsets, const void* g,
                                   const void* u, const void* h, const void* dyp, int E, int R,
                                   int d, int F, void* dg, void* du, void* dxp, void* dw_gate,
                                   void* dw_up, void* dw_down) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, R, d, F, MOE_MXFP8, "moe_grouped_ffn_bwd_mxp");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp, R == 0);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, g, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, u, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, h, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dyp, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dg, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, du, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dxp, R == 0);
  MOE_REQUIRE_PTR(ctx, dw_gate);
  MOE_REQUIRE_PTR(ctx, dw_up);
  MOE_REQUIRE_PTR(ctx, dw_down);
  {
    const size_t rf = (size_t)R * F * 2, w = (size_t)E * d * F * 2;
    MOE_REQUIRE_DISJOINT(ctx, "moe_grouped_ffn_bwd_mxp", {dg, rf, "dg"}, {du, rf, "du"},
                         {dxp, (size_t)R * d * 2, "dxp"}, {dw_gate, w, "dw_gate"}, {dw_up, w, "dw_up"},
                         {dw_down, w, "dw_down"});
  }
  MxWeights w;
  st = pack_regions(ctx, pack, pack_bytes, E, d, F, "moe_grouped_ffn_bwd_mxp", &w);
  if (st != MOE_OK) return st;
  return moe_internal_ffn_bwd_mx(ctx, (const bf16_t*)xp, nullptr, nullptr, nullptr, &w, offsets,
                                 (const bf16_t*)g, (const bf16_t*)u, (const bf16_t*)h,
                                 (const bf16_t*)dyp, E, R, d, F, (bf16_t*)dg, (bf16_t*)du,
                                 (bf16_t*)dxp, (bf16_t*)dw_gate, (bf16_t*)dw_up, (bf16_t*)dw_down, false);
}

moe_status moe_grouped_ffn_bwd_mxp_bf16w(moe_ctx* ctx, const void* xp, const void* pack,
                                         size_t pack_bytes, const int32_t* offsets, const void* g,
                                         const void* u, const void* h, const void* dyp, int E, int R,
                                         int d, int F, void* dg, void* du, void* dxp, void* dw_gate,
                                         void* dw_up, void* dw_down) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, R, d, F, MOE_MXFP8, "moe_grouped_ffn_bwd_mxp_bf16w");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp, R == 0);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, g, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, u, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, h, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dyp, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dg, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, du, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dxp, R == 0);
  MOE_REQUIRE_PTR(ctx, dw_gate);
  MOE_REQUIRE_PTR(ctx, dw_up);
  MOE_REQUIRE_PTR(ctx, dw_down);
  {
    const size_t rf = (size_t)R * F * 2, w = (size_t)E * d * F * 2;
    MOE_REQUIRE_DISJOINT(ctx, "moe_grouped_ffn_bwd_mxp_bf16w", {dg, rf, "dg"}, {du, rf, "du"},
                         {dxp, (size_t)R * d * 2, "dxp"}, {dw_gate, w, "dw_gate"}, {dw_up, w, "dw_up"},
                         {dw_down, w, "dw_down"});
  }
  MxWeights w;
  st = pack_regions(ctx, pack, pack_bytes, E, d, F, "moe_grouped_ffn_bwd_mxp_bf16w", &w);
  if (st != MOE_OK) return st;
  return moe_internal_ffn_bwd_mx(ctx, (const bf16_t*)xp, nullptr, nullptr, nullptr, &w, offsets,
                                 (const bf16_t*)g, (const bf16_t*)u, (const bf16_t*)h,
                                 (const bf16_t*)dyp, E, R, d, F, (bf16_t*)dg, (bf16_t*)du,
                                 (bf16_t*)dxp, (bf16_t*)dw_gate, (bf16_t*)dw_up, (bf16_t*)dw_down, true);
}

static moe_status ffn_bwd_impl(moe_ctx* ctx, const void* xp, const void* w_gate,
                               const void* w_up, const void* w_down, const int32_t* offsets,
                               const void* g, const void* u, const void* h, const void* dyp,
                               int E, int R, int d, int F, moe_dtype dtype, void* dg, void* du,
                               void* dxp, void* dw_gate, void* dw_up, void* dw_down,
                               const float* dl_rows, const void* rw) {
  MOE_CHECK_CTX(ctx);
  moe_status st = ffn_validate(ctx, E, R, d, F, dtype, "moe_grouped_ffn_bwd");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp, R == 0);
  MOE_REQUIRE_PTR(ctx, w_gate);
  MOE_REQUIRE_PTR(ctx, w_up);
  MOE_REQUIRE_PTR(ctx, w_down);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, g, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, u, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, h, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dyp, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dg, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, du, R == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dxp, R == 0);
  MOE_REQUIRE_PTR(ctx, dw_gate);
  MOE_REQUIRE_PTR(ctx, dw_up);
  MOE_REQUIRE_PTR(ctx, dw_down);
  {
    const size_t es = dtype == MOE_F32 ? 4 : 2, rf = (size_t)R * F * es, w = (size_t)E * d * F * es;
    MOE_REQUIRE_DISJOINT(ctx, "moe_grouped_ffn_bwd", {dg, rf, "dg"}, {du, rf, "du"},
                         {dxp, (size_t)R * d * es, "dxp"}, {dw_gate, w, "dw_gate"}, {dw_up, w, "dw_up"},
                         {dw_down, w, "dw_down"});
  }
  if (dtype == MOE_MXFP8)
    return moe_internal_ffn_bwd_mx(ctx, (const bf16_t*)xp, (const bf16_t*)w_gate,
                                   (const bf16_t*)w_up, (const bf16_t*)w_down, nullptr, offsets,
                                   (const bf16_t*)g, (const bf16_t*)u, (const bf16_t*)h,
                                   (const bf16_t*)dyp, E, R, d, F, (bf16_t*)dg, (bf16_t*)du,
                                   (bf16_t*)dxp, (bf16_t*)dw_gate, (bf16_t*)dw_up,
                                   (bf16_t*)dw_down, false);
  if (dtype == MOE_F32)
    return moe_internal_ffn_bwd_f32(ctx, (const float*)xp, (const float*)w_gate,
                                    (const float*)w_up, (const float*)w_down, offsets,
                                    (const float*)g, (const float*)u, (const float*)h,
                                    (const float*)dyp, E, R, d, F, (float*)dg, (float*)du,
                                    (float*)dxp, (float*)dw_gate, (float*)dw_up, (float*)dw_down);
  size_t part_bytes = 0;
  const size_t need = kPlanBytes + wgrad_split_bytes(E, R, d, F, &part_bytes);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "moe_grouped_ffn_bwd: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  int32_t* plan_dn = (int32_t*)ctx->ws;  // XCD ranges of the down wgrad
  int32_t* plan_up = plan_dn + 16;       // and of the gate/up wgrad
  float* split_part = (float*)((char*)ctx->ws + kPlanBytes);
  int32_t* split_voff = (int32_t*)((char*)ctx->ws + kPlanBytes + part_bytes);
  const int dn_per_e = ((d + BN - 1) / BN) * ((F + CfgWD::BM - 1) / CfgWD::BM);
  const int up_per_e = ((F + 127) / 128) * ((d + CfgWU::BM - 1) / CfgWU::BM);
  static_assert(CfgWD::BK == kWgradBK && CfgWU::BK == kWgradBK, "weight-gradient plans use kWgradBK");
  // the down dgrad (R > 0) plans both weight gradients' XCD ranges; with no
  // rows every tile costs the same and equal counts are exact
  const bool planned = R > 0;
  hipError_t e;
  if (R > 0) {
    // down dgrad with the SwiGLU backward in the epilogue
    Params p{};
    p.a0 = (const bf16_t*)dyp;
    p.lda = d;
    p.b0 = (const bf16_t*)w_down;  // B[k=c][n=f] = Wd[f][c]: rows of Wd are K-contiguous
    p.ldb = d;
    p.b_gstride = (long long)F * d;
    p.c0 = dg;
    p.c1 = du;
    p.ldc = F;
    p.aux0 = (const bf16_t*)g;
    p.aux1 = (const bf16_t*)u;
    p.offsets = offsets;
    p.E = E;
    p.N = F;
    p.K = d;
    p.kseg = d;
    p.ntiles = (F + BN - 1) / BN;
    p.xr_out0 = plan_dn;
    p.xr_out1 = plan_up;
    p.xr_pe0 = dn_per_e;
    p.xr_pe1 = up_per_e;
    {
      moe_prof_scope ps(ctx, MOE_K_GEMM_DGRAD_DOWN);
      e = launch_mragged<DGRAD_DOWN>(p, R, ctx->stream);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "down dgrad: %s", hipGetErrorString(e));
  }
  st = run_wgrad_down(ctx, h, dyp, offsets, E, R, d, F, dw_down, plan_dn, planned, split_part, split_voff);
  if (st != MOE_OK) return st;
  if (R > 0) {
    // gate/up dgrad: dxp = dg Wg^T + du Wu^T (K = 2F in two segments)
    Params p{};
    p.a0 = (const bf16_t*)dg;
    p.a1 = (const bf16_t*)du;
    p.lda = F;
    p.b0 = (const bf16_t*)w_gate;  // B[k=f][n=i] = Wg[i][f]: rows of Wg are K-contiguous
    p.b1 = (const bf16_t*)w_up;
    p.ldb = F;
    p.b_gstride = (long long)d * F;
    p.c0 = dxp;
    p.ldc = d;
    p.offsets = offsets;
    p.E = E;
    p.N = d;
    p.K = 2 * F;
    p.kseg = F;
    p.rdl = dl_rows;
    p.rw = (const bf16_t*)rw;
    p.ntiles = (d + BN - 1) / BN;
    {
      moe_prof_scope ps(ctx, MOE_K_GEMM_DGRAD_UP);
      e = launch_mragged<DGRAD_UP>(p, R, ctx->stream);
    }
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "gate/up dgrad: %s", hipGetErrorString(e));
  }
  return run_wgrad_up(ctx, xp, dg, du, offsets, E, R, d, F, dw_gate, dw_up, plan_up, planned, split_part,
                      split_voff);
}

moe_status moe_grouped_ffn_bwd(moe_ctx* ctx, const void* xp, const void* w_gate,
                               const void* w_up, const void* w_down, const int32_t* offsets,
                               const void* g, const void* u, const void* h, const void* dyp,
                               int E, int R, int d, int F, moe_dtype dtype, void* dg, void* du,
                               void* dxp, void* dw_gate, void* dw_up, void* dw_down) {
  return ffn_bwd_impl(ctx, xp, w_gate, w_up, w_down, offsets, g, u, h, dyp, E, R, d, F, dtype, dg,
                      du, dxp, dw_gate, dw_up, dw_down, nullptr, nullptr);
}

moe_status moe_grouped_ffn_bwd_router(moe_ctx* ctx, const void* xp, const void* w_gate,
                                      const void* w_up, const void* w_down,
                                      const int32_t* offsets, const void* g, const void* u,
                                      const void* h, const void* dyp,
                                      const float* dl_rows, const void* w_router, int E, int R,
                                      int d, int F, moe_dtype dtype, void* dg, void* du,
                                      void* dxp, void* dw_gate, void* dw_up, void* dw_down) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, dtype == MOE_BF16, "moe_grouped_ffn_bwd_router: bf16 only");
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dl_rows, R == 0);
  MOE_REQUIRE_PTR(ctx, w_router);
  return ffn_bwd_impl(ctx, xp, w_gate, w_up, w_down, offsets, g, u, h, dyp, E, R, d, F, dtype, dg,
                      du, dxp, dw_gate, dw_up, dw_down, dl_rows, w_router);
}

}  // extern "C"
