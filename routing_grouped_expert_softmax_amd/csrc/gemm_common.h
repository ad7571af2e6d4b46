// gemm_common.h — pieces shared by the bf16 and MXFP8 grouped GEMM kernels:
// the GEMM modes, device-side work finding from the per-expert offsets, the
// LDS-direct loads, and the fused epilogue that stores one block tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe_gemm {

using moe::bf16_t;
using moe::pack2bf;
using moe::sigmoid_f;
using moe::silu_f;

constexpr int BN = 256;        // block tile columns
constexpr int kThreads = 256;  // four waves (the threads that take part in the tile scans)

#define LDS_AS __attribute__((address_space(3)))

enum Mode : int {
  FWD_UP = 0,      // g,u,h = swiglu(xp Wg, xp Wu)            M-ragged, dual B, B N-contig
  FWD_DOWN = 1,    // yp = h Wd                               M-ragged, B N-contig
  DGRAD_DOWN = 2,  // dh = dyp Wd^T -> dg, du                  M-ragged, B K-contig
  DGRAD_UP = 3,    // dxp = dg Wg^T + du Wu^T (two K segments) M-ragged, B K-contig
  WGRAD_UP = 4,    // dWg, dWu = xp^T (dg | du)                K-ragged, dual B
  WGRAD_DOWN = 5,  // dWd = h^T dyp                            K-ragged
  ROUTER = 6       // logits = x W_r (one group, fp32 out)     M = T, B N-contig
};

template <int MODE>
struct Traits {
  static constexpr bool kA_KCONTIG = !(MODE == WGRAD_UP || MODE == WGRAD_DOWN);
  static constexpr bool kB_KCONTIG = (MODE == DGRAD_DOWN || MODE == DGRAD_UP);
  static constexpr bool kDUAL = (MODE == FWD_UP || MODE == WGRAD_UP);
  static constexpr bool kKRAGGED = (MODE == WGRAD_UP || MODE == WGRAD_DOWN);
  static constexpr bool kSINGLE = (MODE == ROUTER);
};


// Work description of one block.
struct Work {
  int e;         // expert (group)
  int row0;      // first A row of the tile (M-ragged) / first K row of the group
  int rows;      // valid rows of the tile (M-ragged) / K length of the group (K-ragged)
  int m0;        // first output M index (K-ragged)
  int nt;        // n-tile
};

// Exclusive block scan of one count per thread over the first kThreads
// threads (the others pass 0 and get the total): an inclusive scan within
// each wave by shuffles, then the kThreads / 64 wave totals through LDS
// (sh[0 .. kThreads/64)), two barriers.  Every thread of the block calls it.
__device__ __forceinline__ void block_excl_scan(int local, int* sh, int& excl, int& total) {
  const int tid = threadIdx.x;
  const bool act = tid < kThreads;
  const int lane = tid & 63, wid = tid >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (act && lane == 63) sh[wid] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int wv = 0; wv < kThreads / 64; ++wv) {
    const int v = sh[wv];
    tot += v;
    if (wv < wid) before += v;
  }
  total = __builtin_amdgcn_readfirstlane(tot);
  excl = act ? before + incl - local : total;
  __syncthreads();
}

// Block-wide search of (expert, tile) for logical tile L in an M-ragged launch.
// Returns false when L is past the real total.
// Tile of a one-tile-per-block row-ragged launch: expert e owns
// ceil(n_e / BM) * ntiles logical tiles (m-tile fastest, experts in order),
// split into eight contiguous ranges, one per XCD.  Returns false for blocks
// past the last tile.
template <int BM>
__device__ bool find_mtile(int E, const int32_t* offsets, int ntiles, int* sh, Work& w) {
  // the first kThreads threads hold the experts; any further threads of a
  // larger block only take part in the barriers
  const int tid = threadIdx.x;
  const int per = (E + kThreads - 1) / kThreads;  // experts per thread (<= 4)
  int cnt[4], til[4];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * per + q;
    cnt[q] = 0;
    til[q] = 0;
    if (q < per && e < E) {
      cnt[q] = offsets[e + 1] - offsets[e];
      til[q] = ((cnt[q] + BM - 1) / BM) * ntiles;
    }
    local += til[q];
  }
  // exclusive scan of `local` over the block
  int run, total;
  block_excl_scan(local, sh, run, total);
  // logical tile of this block: contiguous ranges per XCD
  const int per_xcd = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  const int L = (blockIdx.x & 7) * per_xcd + slot;
  const bool live = slot < per_xcd && L < total;
  if (tid == 0) sh[kThreads] = -1;
  __syncthreads();
  if (live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * per + q;
      if (q < per && e < E && til[q] > 0 && L >= run && L < run + til[q]) {
        const int mt_e = (cnt[q] + BM - 1) / BM;
        const int local_t = L - run;
        sh[kThreads] = e;
        sh[kThreads + 1] = local_t % mt_e;  // m-tile
        sh[kThreads + 2] = local_t / mt_e;  // n-tile
      }
      run += til[q];
    }
  }
  __syncthreads();
  // values read back from LDS are block-uniform: keep them in scalar registers
  const int e = __builtin_amdgcn_readfirstlane(sh[kThreads]);
  if (e < 0) return false;
  const int mt = __builtin_amdgcn_readfirstlane(sh[kThreads + 1]);
  w.e = e;
  w.nt = __builtin_amdgcn_readfirstlane(sh[kThreads + 2]);
  const int beg = offsets[e], end = offsets[e + 1];
  w.row0 = beg + mt * BM;
  w.rows = min(BM, end - w.row0);
  w.m0 = 0;
  return true;
}

// Barrier without a memory fence: waits only for this wave's LDS traffic, so
// output stores still in flight are not drained (a fence would wait for them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// XCD ranges of a K-ragged (wgrad) launch.  Every expert owns per_e output
// tiles (expert-major order); a tile of expert e costs ceil(n_e / BK) + 2 K
// steps (the 2 stand for its prologue and its stores), so the experts' costs
// differ as much as their row counts.  XCD x takes the tiles whose cost
// midpoint lies in [x C/8, (x+1) C/8), C the total cost: eight contiguous
// ranges of nearly equal cost, so one hot expert's tiles spread over several
// XCDs instead of loading one.  Sets [first, end) of this block's XCD; the
// caller's blocks loop over ranges longer than their slots.
template <int BK>
__device__ void kragged_xcd_range(const int32_t* offsets, int E, int per_e, int xcd, int& first,
                                  int& end) {
  // every wave computes the same result with shuffles: no LDS, no barrier
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;  // experts per lane (<= 16)
  int cq[16];                     // K-step cost of this lane's experts
  long long local = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = lane * per + q;
    cq[q] = (q < per && e < E) ? (offsets[e + 1] - offsets[e] + BK - 1) / BK + 2 : 0;
    local += (long long)cq[q] * per_e;
  }
  long long incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const long long C = __shfl(incl, 63, 64);
  const long long P0 = incl - local;  // cost before this lane's first expert
  // Equal tile counts per XCD fill a one-tile-per-block grid exactly; keep
  // them unless their costs are more than 10% out of balance.  The cost of
  // the tiles before tile t = e * per_e + j is P_e + j c_e; P_e and c_e come
  // from the lane that owns expert e.
  const int total = E * per_e, per_xcd = (total + 7) / 8;
  auto cost_before = [&](int t) -> long long {
    if (t >= total) return C;
    const int e = t / per_e, j = t - e * per_e;
    const int owner = e / per, qe = e - owner * per;
    long long pe = P0;
    int ce = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < qe) pe += (long long)cq[q] * per_e;
      if (q == qe) ce = cq[q];
    }
    pe = __shfl(pe, owner, 64);
    ce = __shfl(ce, owner, 64);
    return pe + (long long)j * ce;
  };
  long long worst = 0;
  for (int x = 0; x < 8; ++x) {
    const long long cx =
        cost_before(min((x + 1) * per_xcd, total)) - cost_before(min(x * per_xcd, total));
    worst = cx > worst ? cx : worst;
  }
  // (worst and C are the same in every lane: make the branch wave-uniform)
  if (__builtin_amdgcn_readfirstlane((int)(worst * 80 <= C * 11))) {  // worst <= 1.1 C / 8
    first = __builtin_amdgcn_readfirstlane(min(xcd * per_xcd, total));
    end = __builtin_amdgcn_readfirstlane(min(first + per_xcd, total));
    return;
  }
  // Otherwise tile j of expert e goes to XCD floor(8 * mid / C), mid =
  // P_e + (j + 1/2) c_e.  Counting the tiles below a boundary B in float is
  // exact enough: every block evaluates the same expressions, so the ranges
  // tile [0, E * per_e) without gaps or overlaps, and the count is monotone
  // in B.
  const float b0 = (float)C * (float)xcd * 0.125f, b1 = (float)C * (float)(xcd + 1) * 0.125f;
  int n0 = 0, n1 = 0;
  long long P = P0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (cq[q] > 0) {
      const float pf = (float)P, cf = (float)cq[q];
      auto below = [&](float b) -> int {
        const float n = ceilf((b - pf) / cf - 0.5f);  // j < (B - P) / c - 1/2
        return n <= 0.f ? 0 : (n >= (float)per_e ? per_e : (int)n);
      };
      n0 += below(b0);
      n1 += xcd == 7 ? per_e : below(b1);
      P += (long long)cq[q] * per_e;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    n0 += __shfl_xor(n0, off, 64);
    n1 += __shfl_xor(n1, off, 64);
  }
  first = __builtin_amdgcn_readfirstlane(n0);
  end = __builtin_amdgcn_readfirstlane(n1);
}


// Tile table of a row-ragged launch: expert e owns ceil(n_e / BM) * ntiles
// logical tiles, m-tile fastest, experts in order.  Each thread keeps the
// exclusive scan of the tile counts of its (up to four) experts.
// NFAST: an expert's tiles in m-major order (the n-tiles of one row tile
// consecutive); otherwise n-major (the row tiles sharing one weight tile
// consecutive).
template <int BM, bool NFAST = false>
struct MTileSched {
  int cnt[4], til[4];
  int run;    // first logical tile of this thread's experts
  int per;    // experts per thread
  int total;  // tiles of the launch (block-uniform)
  int ntiles_;
  __device__ void init(int E, const int32_t* offsets, int ntiles, int* sh) {
    ntiles_ = ntiles;
    // threads past kThreads (larger blocks) hold no experts
    const int tid = threadIdx.x;
    per = (E + kThreads - 1) / kThreads;  // <= 4
    int local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * per + q;
      cnt[q] = 0;
      til[q] = 0;
      if (q < per && e < E) {
        cnt[q] = offsets[e + 1] - offsets[e];
        til[q] = ((cnt[q] + BM - 1) / BM) * ntiles;
      }
      local += til[q];
    }
    block_excl_scan(local, sh, run, total);
  }
  // Work of logical tile L < total.  The owning thread publishes it through
  // sh[kThreads..+2]; the caller keeps a barrier between one call's reads and
  // the next call's write (every K step has one).
  __device__ void lookup(int L, const int32_t* offsets, int* sh, Work& w) const {
    const int tid = threadIdx.x;
    int r = run;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * per + q;
      if (q < per && til[q] > 0 && L >= r && L < r + til[q]) {
        const int mt_e = (cnt[q] + BM - 1) / BM;
        const int local_t = L - r;
        sh[kThreads] = e;
        if (NFAST) {
          const int nt = ntiles_;
          sh[kThreads + 1] = local_t / nt;  // m-tile
          sh[kThreads + 2] = local_t % nt;  // n-tile
        } else {
          sh[kThreads + 1] = local_t % mt_e;  // m-tile
          sh[kThreads + 2] = local_t / mt_e;  // n-tile
        }
      }
      r += til[q];
    }
    lds_barrier();
    // block-uniform values: keep them in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(sh[kThreads]);
    const int mt = __builtin_amdgcn_readfirstlane(sh[kThreads + 1]);
    w.e = e;
    w.nt = __builtin_amdgcn_readfirstlane(sh[kThreads + 2]);
    const int beg = offsets[e], end = offsets[e + 1];
    w.row0 = beg + mt * BM;
    w.rows = min(BM, end - w.row0);
    w.m0 = 0;
  }
};


// Raw buffer descriptor (V#) of `bytes` bytes at `base`: dword0/1 base address
// (stride 0), dword2 the range in bytes (loads past it return zero), dword3
// the gfx9 data-format word.  Built from scalar values (every lane computes
// the same base), so the descriptor lives in SGPRs as the loads require.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned long long bytes) {
  const unsigned long long a = (unsigned long long)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)(unsigned)(bytes > 0xffffffffull ? 0xffffffffull : bytes));
  r[3] = 0x00020000;
  return r;
}

// 16-byte-per-lane buffer load straight into LDS (lane l writes lds + 16*l).
// Issued as inline assembly so the compiler's wait-count pass does not treat
// it as an LDS write that every later LDS read must wait for: the kernel
// waits for these loads itself (s_waitcnt vmcnt) before the barrier that
// publishes a stage.  The instruction has no register outputs.  M0 carries
// the LDS address (one wait state between writing M0 and the load) and is
// declared clobbered, so the compiler keeps nothing of its own in M0 across
// the statement.
__device__ __forceinline__ void dma16(rsrc_t r, LDS_AS void* lds, int voff,
                                      int soff) {
  const unsigned lds_addr = (unsigned)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

// 4-byte-per-lane variant (lane l writes lds + 4*l), for block-scale rows.
__device__ __forceinline__ void dma4(rsrc_t r, LDS_AS void* lds, int voff, int soff) {
  const unsigned lds_addr = (unsigned)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

// Output description for the epilogue.
struct EpiArgs {
  void* c0;
  void* c1;
  void* c2;
  int ldc;
  long long c_gstride;
  const bf16_t* aux0;
  const bf16_t* aux1;
  int N;
  int M;
};

// Direct epilogue: every lane stores its own 4-column pieces straight from
// the accumulators (each store covers 16 bytes of 32 rows), used where the
// staging regions below do not fit.  Lane holds
// C[m = mbase + (lane&31)][n = nbase + 8*(r/4) + 4*(lane>>5) + r%4] of each
// 32x32 subtile; dual modes hold g (subtiles 0,1) and u (2,3) of the same
// columns.
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int MODE, int BM, int SM, bool SWIGLU_FROM_BF16, int SN = 4, int WN = 128>
__device__ __forceinline__ void store_tile_direct(const f32x16 (&acc)[SM][SN], const EpiArgs& a,
                                                  const Work& w, int lane, int wm, int wn) {
  constexpr int WM = SM * 32;  // wave tile rows
  // Lane holds C[m = mbase + (lane&31)][n = nbase + 8*(r/4) + 4*(lane>>5) + r%4].
  const int ncol4 = 4 * (lane >> 5);
#pragma unroll
  for (int sm = 0; sm < SM; ++sm) {
    const int mloc = wm * WM + sm * 32 + (lane & 31);  // row inside the block tile
    bool mvalid;
    size_t crow;
    if (Traits<MODE>::kKRAGGED) {
      mvalid = (w.m0 + mloc) < a.M;
      crow = (size_t)(w.m0 + mloc);
    } else {
      mvalid = mloc < w.rows;
      crow = (size_t)(w.row0 + mloc);
    }
    if (!mvalid) continue;
    if (Traits<MODE>::kDUAL) {
#pragma unroll
      for (int sn = 0; sn < SN / 2; ++sn) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = w.nt * 128 + wn * (WN / 2) + sn * 32 + 8 * g4 + ncol4;
          if (col >= a.N) continue;
          float gv[4], uv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gv[r] = acc[sm][sn][g4 * 4 + r];
            uv[r] = acc[sm][sn + SN / 2][g4 * 4 + r];
          }
          if (MODE == FWD_UP) {
            const size_t off = crow * a.ldc + col;
            *reinterpret_cast<uint2*>((bf16_t*)a.c0 + off) =
                make_uint2(pack2bf(gv[0], gv[1]), pack2bf(gv[2], gv[3]));
            *reinterpret_cast<uint2*>((bf16_t*)a.c1 + off) =
                make_uint2(pack2bf(uv[0], uv[1]), pack2bf(uv[2], uv[3]));
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gg = SWIGLU_FROM_BF16 ? moe::bf2f(moe::f2bf(gv[r])) : gv[r];
              const float uu = SWIGLU_FROM_BF16 ? moe::bf2f(moe::f2bf(uv[r])) : uv[r];
              hv[r] = silu_f(gg) * uu;
            }
            *reinterpret_cast<uint2*>((bf16_t*)a.c2 + off) =
                make_uint2(pack2bf(hv[0], hv[1]), pack2bf(hv[2], hv[3]));
          } else {  // WGRAD_UP
            const size_t off = (size_t)w.e * a.c_gstride + crow * a.ldc + col;
            *reinterpret_cast<uint2*>((bf16_t*)a.c0 + off) =
                make_uint2(pack2bf(gv[0], gv[1]), pack2bf(gv[2], gv[3]));
            *reinterpret_cast<uint2*>((bf16_t*)a.c1 + off) =
                make_uint2(pack2bf(uv[0], uv[1]), pack2bf(uv[2], uv[3]));
          }
        }
      }
    } else {
#pragma unroll
      for (int sn = 0; sn < SN; ++sn) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = w.nt * BN + wn * WN + sn * 32 + 8 * g4 + ncol4;
          if (col >= a.N) continue;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[sm][sn][g4 * 4 + r];
          if (MODE == ROUTER) {
            if (a.aux0 != nullptr) {
              // add into a bf16 matrix: c0 = aux0 + tile, one rounding (c0 may be aux0)
              const size_t off = crow * a.ldc + col;
              const uint2 raw = *reinterpret_cast<const uint2*>(a.aux0 + off);
              const uint32_t w[2] = {raw.x, raw.y};
              float s[4];
#pragma unroll
              for (int r = 0; r < 4; ++r)
                s[r] = __uint_as_float((r & 1) ? (w[r >> 1] & 0xffff0000u) : (w[r >> 1] << 16)) + v[r];
              *reinterpret_cast<uint2*>((bf16_t*)a.c0 + off) = make_uint2(pack2bf(s[0], s[1]), pack2bf(s[2], s[3]));
            } else {
              float* c = (float*)a.c0 + crow * a.ldc + col;
              *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
            }
          } else if (MODE == DGRAD_DOWN) {
            const size_t off = crow * a.ldc + col;
            const uint2 graw = *reinterpret_cast<const uint2*>(a.aux0 + off);
            const uint2 uraw = *reinterpret_cast<const uint2*>(a.aux1 + off);
            const uint32_t gw[2] = {graw.x, graw.y}, uw[2] = {uraw.x, uraw.y};
            float dg[4], du[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = __uint_as_float((r & 1) ? (gw[r >> 1] & 0xffff0000u) : (gw[r >> 1] << 16));
              const float u = __uint_as_float((r & 1) ? (uw[r >> 1] & 0xffff0000u) : (uw[r >> 1] << 16));
              const float s = sigmoid_f(g);
              dg[r] = v[r] * u * s * (1.0f + g * (1.0f - s));
              du[r] = v[r] * g * s;
            }
            *reinterpret_cast<uint2*>((bf16_t*)a.c0 + off) =
                make_uint2(pack2bf(dg[0], dg[1]), pack2bf(dg[2], dg[3]));
            *reinterpret_cast<uint2*>((bf16_t*)a.c1 + off) =
                make_uint2(pack2bf(du[0], du[1]), pack2bf(du[2], du[3]));
          } else {
            size_t off = crow * a.ldc + col;
            if (Traits<MODE>::kKRAGGED) off += (size_t)w.e * a.c_gstride;
            *reinterpret_cast<uint2*>((bf16_t*)a.c0 + off) =
                make_uint2(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]));
          }
        }
      }
    }
  }
}


// Split-K partials of a K-ragged (wgrad) tile: every lane stores its own
// 4-column fp32 pieces of group w.e's partial product, exact (no rounding),
// for a fixed-order reduction into the bf16 weight gradient.  Dual modes
// write g columns (subtiles 0,1) to c0 and u columns (2,3) to c1.
template <int MODE, int BM, int SM, int SN = 4, int WN = 128>
__device__ __forceinline__ void store_partial_f32(const f32x16 (&acc)[SM][SN], const EpiArgs& a,
                                                  const Work& w, int lane, int wm, int wn) {
  static_assert(Traits<MODE>::kKRAGGED, "split-K partials are for the K-ragged modes");
  constexpr int WM = SM * 32;  // wave tile rows
  const int ncol4 = 4 * (lane >> 5);
  const size_t gbase = (size_t)w.e * a.c_gstride;
#pragma unroll
  for (int sm = 0; sm < SM; ++sm) {
    const int m = w.m0 + wm * WM + sm * 32 + (lane & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = Traits<MODE>::kDUAL
                            ? w.nt * 128 + wn * (WN / 2) + (sn % (SN / 2)) * 32 + 8 * g4 + ncol4
                            : w.nt * BN + wn * WN + sn * 32 + 8 * g4 + ncol4;
        if (col >= a.N) continue;
        float* out = (float*)(Traits<MODE>::kDUAL && sn >= SN / 2 ? a.c1 : a.c0);
        const f32x4 v = {acc[sm][sn][g4 * 4], acc[sm][sn][g4 * 4 + 1], acc[sm][sn][g4 * 4 + 2],
                         acc[sm][sn][g4 * 4 + 3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + gbase + (size_t)m * a.ldc + col));
      }
    }
  }
}

// Epilogue staging region of a wave: inside stage buffer wave / PER at
// offset (wave % PER) * REG, where PER regions fit in one stage buffer.
// Callers static_assert that S * PER >= 4.
// Epilogue staging.  Each wave owns a private LDS region (inside the stage
// buffers, free once the main loop's last barrier has passed) and writes its
// outputs through it CH rows at a time: accumulators go into LDS in the MFMA
// layout, then every lane reads 16 contiguous bytes of a row and stores them,
// so each store instruction writes whole row segments instead of 16 bytes in
// each of 32 rows.  The down dgrad reads the saved g and u the same way in
// reverse.  Rows of a region are WNO bf16 wide; 16-byte chunks are XOR-
// swizzled with the row so that column-wise MFMA-layout writes and row-wise
// reads both spread over the banks.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 bf4(const float (&v)[4]) {
  u32x2 r;
  r.x = pack2bf(v[0], v[1]);
  r.y = pack2bf(v[2], v[3]);
  return r;
}

template <int MODE>
constexpr int epi_nout() {
  return MODE == FWD_UP ? 3 : (Traits<MODE>::kDUAL || MODE == DGRAD_DOWN) ? 2 : 1;
}
// Staged row width: a wave's 128 output columns (64 per matrix in the dual
// modes), or half of them per pass when the region must shrink (NCS = 2).
template <int MODE>
constexpr int epi_wno(int ncs) { return Traits<MODE>::kDUAL ? 64 : 128 / ncs; }
template <int MODE>
constexpr int epi_region_bytes(int ch, int ncs) {
  return epi_nout<MODE>() * ch * epi_wno<MODE>(ncs) * 2;
}
// Column passes of the staged epilogue: 1 or 2 (whichever lets the NW wave
// regions of 32 rows fit in the stage buffers), 0 = direct epilogue.
template <int MODE, int NW = 4>
constexpr int epi_ncs(int stage_bytes, int stages) {
  if (MODE == ROUTER) return 0;
  // the down dgrad prefetches g and u of the next chunk into registers: two
  // 64-column passes keep that prefetch at 32 VGPRs per lane
  if (MODE == DGRAD_DOWN && stages * (stage_bytes / epi_region_bytes<MODE>(32, 2)) >= NW) return 2;
  if (stages * (stage_bytes / epi_region_bytes<MODE>(32, 1)) >= NW) return 1;
  if (!Traits<MODE>::kDUAL && stages * (stage_bytes / epi_region_bytes<MODE>(32, 2)) >= NW) return 2;
  return 0;
}
template <int MODE, int NW = 4>
constexpr bool epi_staged(int stage_bytes, int stages) { return epi_ncs<MODE, NW>(stage_bytes, stages) > 0; }
// Rows per chunk: 64 when the NW wave regions fit in the stage buffers, else 32.
template <int MODE, int NW = 4>
constexpr int epi_chunk(int stage_bytes, int stages) {
  if (MODE == DGRAD_DOWN) return 32;  // register budget of the g, u prefetch
  return stages * (stage_bytes / epi_region_bytes<MODE>(64, epi_ncs<MODE, NW>(stage_bytes, stages))) >= NW
             ? 64
             : 32;
}

// Stores one block tile.  Lane holds
// C[m = mbase + (lane&31)][n = nbase + 8*(r/4) + 4*(lane>>5) + r%4] of each
// 32x32 subtile; dual modes hold g (subtiles 0,1) and u (2,3) of the same
// columns.  SWIGLU_FROM_BF16: the forward's h (and the dgrad's silu terms)
// are computed from the bf16-rounded g and u instead of the fp32 sums.
// wbuf: this wave's staging region, epi_region_bytes<MODE>(CH, NCS) bytes.
// OPAQUE: recompute the lane's staging addresses per tile instead of letting
// the compiler keep them live through the main loop (where registers are
// short they would be spilled and reloaded before every staged row).
template <int MODE, int BM, int SM, bool SWIGLU_FROM_BF16, int CH, int NCS = 1, bool OPAQUE = false>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[SM][4], const EpiArgs& a,
                                           const Work& w, int lane, int wm, int wn,
                                           LDS_AS unsigned char* wbuf) {
  if constexpr (OPAQUE) asm volatile("" : "+v"(lane));
  constexpr int WM = SM * 32;  // wave tile rows
  const int ncol4 = 4 * (lane >> 5);
  if constexpr (MODE == ROUTER) {
    // fp32 scores, E columns: direct stores (small output)
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
      const int mloc = wm * WM + sm * 32 + (lane & 31);
      if (mloc >= w.rows) continue;
      const size_t crow = (size_t)(w.row0 + mloc);
#pragma unroll
      for (int sn = 0; sn < 4; ++sn)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = w.nt * BN + wn * 128 + sn * 32 + 8 * g4 + ncol4;
          if (col >= a.N) continue;
          float* c = (float*)a.c0 + crow * a.ldc + col;
          *reinterpret_cast<float4*>(c) = make_float4(acc[sm][sn][g4 * 4], acc[sm][sn][g4 * 4 + 1],
                                                      acc[sm][sn][g4 * 4 + 2], acc[sm][sn][g4 * 4 + 3]);
        }
    }
    return;
  } else {
    constexpr bool DUAL = Traits<MODE>::kDUAL;
    static_assert(!DUAL || NCS == 1, "dual epilogues stage all columns at once");
    constexpr int WNO = epi_wno<MODE>(NCS);
    constexpr int SNH = 4 / NCS;        // 32-column subtiles per pass (non-dual)
    constexpr int NOUT = epi_nout<MODE>();
    constexpr int PITCH = WNO * 2;      // bytes per staged row
    constexpr int CPR = PITCH / 16;     // 16-byte chunks per row
    constexpr int MAT = CH * PITCH;     // bytes per staged matrix
    constexpr int RPI = 1024 / PITCH;   // rows per wave-wide 16-byte access
    constexpr int SMC = CH / 32;
    static_assert(WM % CH == 0, "chunk must divide the wave tile");
    const int colw = DUAL ? w.nt * 128 + wn * 64 : w.nt * BN + wn * 128;  // wave's first column
    const size_t gbase = Traits<MODE>::kKRAGGED ? (size_t)w.e * a.c_gstride : 0;
    // staged byte offset of (row, 4-column group) in MFMA layout
    auto frag_off = [&](int row, int col) {
      return row * PITCH + (((col >> 3) ^ (row & (CPR - 1))) << 4) + (((col >> 2) & 1) << 3);
    };
    // row-wise access: lane -> (row within the access, chunk)
    const int rw_row = lane / CPR, rw_chunk = lane % CPR;
    auto row_ok = [&](int mloc, size_t& crow) {
      if (Traits<MODE>::kKRAGGED) {
        crow = (size_t)(w.m0 + mloc);
        return (w.m0 + mloc) < a.M;
      }
      crow = (size_t)(w.row0 + mloc);
      return mloc < w.rows;
    };
    // Down dgrad: the saved g, u rows of each (chunk, pass) are loaded one
    // iteration ahead (coalesced 16-byte loads into registers), so only the
    // first iteration waits for HBM.
    constexpr int NGU = MODE == DGRAD_DOWN ? CH / RPI : 1;
    u32x4 pg[NGU], pu[NGU];
    auto load_gu = [&](int qq, int hh) {
      const int mb = wm * WM + qq * CH, c0 = colw + hh * WNO + rw_chunk * 8;
#pragma unroll
      for (int it = 0; it < NGU; ++it) {
        size_t crow;
        if (row_ok(mb + it * RPI + rw_row, crow) && c0 < a.N) {
          const size_t off = crow * a.ldc + c0;
          pg[it] = *reinterpret_cast<const u32x4*>(a.aux0 + off);
          pu[it] = *reinterpret_cast<const u32x4*>(a.aux1 + off);
        }
      }
    };
    if (MODE == DGRAD_DOWN) load_gu(0, 0);
#pragma unroll
    for (int q = 0; q < WM / CH; ++q)
#pragma unroll
    for (int h = 0; h < NCS; ++h) {
      const int mbase = wm * WM + q * CH;  // first block-tile row of this chunk
      const int col0 = colw + h * WNO;      // first column of this pass
      if (MODE == DGRAD_DOWN) {
        // this iteration's g, u rows -> LDS, then the next iteration's loads
#pragma unroll
        for (int it = 0; it < NGU; ++it) {
          const int row = it * RPI + rw_row;
          size_t crow;
          if (row_ok(mbase + row, crow) && col0 + rw_chunk * 8 < a.N) {
            const int lo = row * PITCH + ((rw_chunk ^ (row & (CPR - 1))) << 4);
            *reinterpret_cast<LDS_AS u32x4*>(wbuf + lo) = pg[it];
            *reinterpret_cast<LDS_AS u32x4*>(wbuf + MAT + lo) = pu[it];
          }
        }
        if (q * NCS + h + 1 < (WM / CH) * NCS) {
          asm volatile("" ::: "memory");
          load_gu(h + 1 < NCS ? q : q + 1, h + 1 < NCS ? h + 1 : 0);
        }
      }
      asm volatile("" ::: "memory");
      // accumulators -> LDS
#pragma unroll
      for (int s = 0; s < SMC; ++s) {
        const int sm = q * SMC + s;
        const int row = s * 32 + (lane & 31);
        if (DUAL) {
#pragma unroll
          for (int sn = 0; sn < 2; ++sn)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int off = frag_off(row, sn * 32 + 8 * g4 + ncol4);
              float gv[4], uv[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                gv[r] = acc[sm][sn][g4 * 4 + r];
                uv[r] = acc[sm][sn + 2][g4 * 4 + r];
              }
              *reinterpret_cast<LDS_AS u32x2*>(wbuf + off) = bf4(gv);
              *reinterpret_cast<LDS_AS u32x2*>(wbuf + MAT + off) = bf4(uv);
              if (MODE == FWD_UP) {
                float hv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const float gg = SWIGLU_FROM_BF16 ? moe::bf2f(moe::f2bf(gv[r])) : gv[r];
                  const float uu = SWIGLU_FROM_BF16 ? moe::bf2f(moe::f2bf(uv[r])) : uv[r];
                  hv[r] = silu_f(gg) * uu;
                }
                *reinterpret_cast<LDS_AS u32x2*>(wbuf + 2 * MAT + off) = bf4(hv);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
          for (int sn = 0; sn < 4; ++sn) {
            if (sn / SNH != h) continue;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int off = frag_off(row, (sn % SNH) * 32 + 8 * g4 + ncol4);
              float v[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = acc[sm][sn][g4 * 4 + r];
              if (MODE == DGRAD_DOWN) {
                const u32x2 gw = *reinterpret_cast<const LDS_AS u32x2*>(wbuf + off);
                const u32x2 uw = *reinterpret_cast<const LDS_AS u32x2*>(wbuf + MAT + off);
                const uint32_t gq[2] = {gw.x, gw.y}, uq[2] = {uw.x, uw.y};
                float dg[4], du[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const float g = __uint_as_float((r & 1) ? (gq[r >> 1] & 0xffff0000u) : (gq[r >> 1] << 16));
                  const float u = __uint_as_float((r & 1) ? (uq[r >> 1] & 0xffff0000u) : (uq[r >> 1] << 16));
                  const float sg = sigmoid_f(g);
                  dg[r] = v[r] * u * sg * (1.0f + g * (1.0f - sg));
                  du[r] = v[r] * g * sg;
                }
                *reinterpret_cast<LDS_AS u32x2*>(wbuf + off) = bf4(dg);
                *reinterpret_cast<LDS_AS u32x2*>(wbuf + MAT + off) = bf4(du);
              } else {
                *reinterpret_cast<LDS_AS u32x2*>(wbuf + off) = bf4(v);
              }
            }
          }
        }
      }
      asm volatile("" ::: "memory");
      // LDS -> global, whole row segments per access
      void* const outs[3] = {a.c0, a.c1, a.c2};
#pragma unroll
      for (int it = 0; it < CH / RPI; ++it) {
        const int row = it * RPI + rw_row;
        size_t crow;
        const int col = col0 + rw_chunk * 8;
        const bool ok = row_ok(mbase + row, crow) && col < a.N;
        const int lo = row * PITCH + ((rw_chunk ^ (row & (CPR - 1))) << 4);
#pragma unroll
        for (int m = 0; m < NOUT; ++m) {
          const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(wbuf + m * MAT + lo);
          // streaming store: the output is not re-read by this kernel
          if (ok)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>((bf16_t*)outs[m] + gbase + crow * a.ldc + col));
        }
      }
      asm volatile("" ::: "memory");
    }
  }
}

}  // namespace moe_gemm
