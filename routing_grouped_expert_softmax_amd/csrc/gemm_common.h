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
constexpr int kThreads = 256;  // four waves

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

// Block-wide search of (expert, tile) for logical tile L in an M-ragged launch.
// Returns false when L is past the real total.
template <int BM>
__device__ bool find_mtile(int E, const int32_t* offsets, int ntiles, int* sh, Work& w) {
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
  sh[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int total = sh[kThreads - 1];
  int run = sh[tid] - local;
  __syncthreads();
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
// the LDS address (one wait state between writing M0 and the load).
__device__ __forceinline__ void dma16(rsrc_t r, LDS_AS void* lds, int voff,
                                      int soff) {
  const unsigned lds_addr = (unsigned)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// 4-byte-per-lane variant (lane l writes lds + 4*l), for block-scale rows.
__device__ __forceinline__ void dma4(rsrc_t r, LDS_AS void* lds, int voff, int soff) {
  const unsigned lds_addr = (unsigned)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory");
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

// Stores one block tile.  Lane holds
// C[m = mbase + (lane&31)][n = nbase + 8*(r/4) + 4*(lane>>5) + r%4] of each
// 32x32 subtile; dual modes hold g (subtiles 0,1) and u (2,3) of the same
// columns.  SWIGLU_FROM_BF16: the forward's h (and the dgrad's silu terms)
// are computed from the bf16-rounded g and u instead of the fp32 sums.
typedef __attribute__((ext_vector_type(16))) float f32x16;
template <int MODE, int BM, int SM, bool SWIGLU_FROM_BF16>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[SM][4], const EpiArgs& a,
                                           const Work& w, int lane, int wm, int wn) {
  constexpr int WM = BM / 2;
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
      for (int sn = 0; sn < 2; ++sn) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = w.nt * 128 + wn * 64 + sn * 32 + 8 * g4 + ncol4;
          if (col >= a.N) continue;
          float gv[4], uv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gv[r] = acc[sm][sn][g4 * 4 + r];
            uv[r] = acc[sm][sn + 2][g4 * 4 + r];
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
      for (int sn = 0; sn < 4; ++sn) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = w.nt * BN + wn * 128 + sn * 32 + 8 * g4 + ncol4;
          if (col >= a.N) continue;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[sm][sn][g4 * 4 + r];
          if (MODE == ROUTER) {
            float* c = (float*)a.c0 + crow * a.ldc + col;
            *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
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

}  // namespace moe_gemm
