// stats.hip — routing statistics, the switch-style load-balance loss and its
// logit gradient, and per-expert weight-gradient norms.
//
// Pages: the load imbalance that a larger expert pool amplifies is why MoE
// frameworks add a load-balancing auxiliary loss ([P2] 2.2, third point);
// the expert heat to watch is the tokens each expert receives, twice the mean
// flagging imbalance ([P2] 4.2); the loss weight starts small ([P2] 4.3);
// the per-expert statistics worth logging are tokens received, mean top-1
// probability and the L2 norms of the expert weight gradients ([P2] 5.2);
// the router supports load balancing ([P1] 四) and a balance score can
// improve while the real load worsens ([P1], negative results), so the real
// counts are always reported beside the loss.
//
// Everything is deterministic: per-lane sums in a fixed token order, wave
// butterflies, and per-block partials added in block order by a second pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>

#include "common.h"

using namespace moe;

namespace {

constexpr int kStatBlocks = 256;      // most partial-sum blocks of one pass
// token rows loaded at once per wave: 32 logits per lane in flight
template <int EPL>
constexpr int rows_in_flight() { return EPL >= 16 ? 2 : 32 / EPL > 16 ? 16 : 32 / EPL; }
constexpr int kNormChunks = 256;      // most partial sums per expert (norms)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// One token's softmax over all E experts, lane l holding experts l + 64 i:
// p[i] = exp(l - max) / sum, inv = 1 / sum (the top-1 probability, since the
// top-1 term is exp(0)), top1 = the lowest expert index holding the largest
// logit.  Lanes past E hold p = 0.
template <int EPL>
__device__ __forceinline__ void token_softmax(const float (&lv)[EPL], int E, int lane, float (&p)[EPL],
                                              float& inv, int& top1) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = fmaxf(m, lv[i]);
  m = wave_max(m);
  int cand = INT_MAX;
#pragma unroll
  for (int i = EPL - 1; i >= 0; --i)
    if (lane + 64 * i < E && lv[i] == m) cand = lane + 64 * i;
  top1 = wave_min(cand);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    p[i] = lane + 64 * i < E ? __expf(lv[i] - m) : 0.f;
    s += p[i];
  }
  inv = 1.0f / wave_sum(s);
#pragma unroll
  for (int i = 0; i < EPL; ++i) p[i] *= inv;
}

template <int EPL>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int E, int lane, float (&lv)[EPL]) {
#pragma unroll
  for (int i = 0; i < EPL; ++i) lv[i] = lane + 64 * i < E ? row[lane + 64 * i] : -INFINITY;
}

// Pass 1 of the statistics: block b covers tokens [b*tpb, (b+1)*tpb), wave w
// the tokens b*tpb + w, +4, ...  Per expert it sums the probabilities, the
// top-1 probabilities and the top-1 counts of its tokens, and writes one
// partial per block, expert-major: part_p, part_s [E][kStatBlocks] fp32,
// part_c [E][kStatBlocks] int32 (entry e * kStatBlocks + b).
template <int EPL>
__global__ void __launch_bounds__(256) stats_partial_kernel(const float* __restrict__ logits, int T_,
                                                            int E, int tpb, float* __restrict__ part_p,
                                                            float* __restrict__ part_s,
                                                            int32_t* __restrict__ part_c) {
  constexpr int U = rows_in_flight<EPL>();
  __shared__ float sp[4][EPL * 64], ss[4][EPL * 64];
  __shared__ int sc[4][EPL * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float ap[EPL], as[EPL];
  int ac[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    ap[i] = 0.f;
    as[i] = 0.f;
    ac[i] = 0;
  }
  const int t0 = blockIdx.x * tpb, t1 = min(T_, t0 + tpb);
  for (int tb = t0 + w; tb < t1; tb += 4 * U) {
    float lv[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + 4 * u;
      if (t < t1) load_row<EPL>(logits + (size_t)t * E, E, lane, lv[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + 4 * u >= t1) break;
      float p[EPL], inv;
      int top1;
      token_softmax<EPL>(lv[u], E, lane, p, inv, top1);
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        ap[i] += p[i];
        if (lane + 64 * i == top1) {
          ac[i] += 1;
          as[i] += inv;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    sp[w][lane + 64 * i] = ap[i];
    ss[w][lane + 64 * i] = as[i];
    sc[w][lane + 64 * i] = ac[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const size_t o = (size_t)e * kStatBlocks + blockIdx.x;
    part_p[o] = ((sp[0][e] + sp[1][e]) + sp[2][e]) + sp[3][e];
    part_s[o] = ((ss[0][e] + ss[1][e]) + ss[2][e]) + ss[3][e];
    part_c[o] = sc[0][e] + sc[1][e] + sc[2][e] + sc[3][e];
  }
}

// Pass 2: one wave per expert adds its nblk partials (lane l takes blocks
// l, l+64, ... in order, then a butterfly), writes the statistics and the
// loss term counts[e] * prob_mean[e] into term[e].
__global__ void __launch_bounds__(256) stats_expert_kernel(
    const float* __restrict__ part_p, const float* __restrict__ part_s,
    const int32_t* __restrict__ part_c, int nblk, const int32_t* __restrict__ counts, int T_, int E,
    float* __restrict__ prob_mean, int32_t* __restrict__ top1_count,
    float* __restrict__ top1_prob_mean, float* __restrict__ term) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= E) return;
  const size_t o = (size_t)e * kStatBlocks;
  float P = 0.f, S = 0.f;
  int C = 0;
#pragma unroll
  for (int j = 0; j < kStatBlocks / 64; ++j) {
    const int b = lane + 64 * j;
    if (b < nblk) {
      P += part_p[o + b];
      S += part_s[o + b];
      C += part_c[o + b];
    }
  }
  P = wave_sum(P);
  S = wave_sum(S);
#pragma unroll
  for (int off = 32; off; off >>= 1) C += __shfl_xor(C, off);
  if (lane == 0) {
    const float pm = T_ > 0 ? P / (float)T_ : 0.f;
    prob_mean[e] = pm;
    top1_count[e] = C;
    top1_prob_mean[e] = C > 0 ? S / (float)C : 0.f;
    term[e] = (float)counts[e] * pm;
  }
}

// Pass 3: the loss, scale * sum_e term[e] by a fixed tree over experts
// (scale = alpha * E / (T * k)).
__global__ void __launch_bounds__(1024) stats_loss_kernel(const float* __restrict__ term, int E,
                                                          float scale, float* __restrict__ aux_loss) {
  __shared__ float red[1024];
  const int e = threadIdx.x;
  red[e] = e < E ? term[e] : 0.f;
  __syncthreads();
  for (int h = 512; h > 0; h >>= 1) {
    if (e < h) red[e] += red[e + h];
    __syncthreads();
  }
  if (e == 0) aux_loss[0] = scale * red[0];
}

// Logit gradient of dloss * aux_loss: with a_e = coef * counts[e]
// (coef = dloss * alpha * E / (T^2 k)), dl[t,e] = p_te (a_e - sum_i p_ti a_i).
// One wave per token, U token rows in flight; every logit is written.
template <int EPL>
__global__ void __launch_bounds__(256) aux_bwd_kernel(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ counts, int T_,
                                                      int E, float coef, float* __restrict__ dl) {
  constexpr int U = rows_in_flight<EPL>();
  const int lane = threadIdx.x & 63;
  float a[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) a[i] = lane + 64 * i < E ? coef * (float)counts[lane + 64 * i] : 0.f;
  const int nw = gridDim.x * 4;
  for (int tb = blockIdx.x * 4 + (threadIdx.x >> 6); tb < T_; tb += nw * U) {
    float lv[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + nw * u;
      if (t < T_) load_row<EPL>(logits + (size_t)t * E, E, lane, lv[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + nw * u;
      if (t >= T_) break;
      float p[EPL], inv;
      int top1;
      token_softmax<EPL>(lv[u], E, lane, p, inv, top1);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) dot += p[i] * a[i];
      dot = wave_sum(dot);
      float* out = dl + (size_t)t * E;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) out[lane + 64 * i] = p[i] * (a[i] - dot);
    }
  }
}

// Sum of squares of chunk c of expert e's n values (16-byte loads, four in
// flight per thread), reduced in a fixed order into part[e][c].
template <typename TE>
__global__ void __launch_bounds__(256) grad_norm_partial_kernel(const TE* __restrict__ dw, size_t n,
                                                                size_t per, float* __restrict__ part) {
  constexpr int V = 16 / sizeof(TE);
  __shared__ float red[4];
  const int c = blockIdx.x, e = blockIdx.y;
  const TE* base = dw + (size_t)e * n;
  const size_t lo = (size_t)c * per, hi = min(n, lo + per);
  float acc = 0.f;
  auto add = [&](const uint4& raw) {
    const TE* v = reinterpret_cast<const TE*>(&raw);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float x = Elem<TE>::ld(v, j);
      acc += x * x;
    }
  };
  size_t i = lo + (size_t)threadIdx.x * V;
  constexpr size_t STEP = 256 * V;
  for (; i + 3 * STEP < hi; i += 4 * STEP) {
    uint4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = *reinterpret_cast<const uint4*>(base + i + j * STEP);
#pragma unroll
    for (int j = 0; j < 4; ++j) add(r[j]);
  }
  for (; i < hi; i += STEP) add(*reinterpret_cast<const uint4*>(base + i));
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[(size_t)e * gridDim.x + c] = ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ void grad_norm_final_kernel(const float* __restrict__ part, int nchunk, int E,
                                       float* __restrict__ norms) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += part[(size_t)e * nchunk + c];
  norms[e] = sqrtf(s);
}

// Tokens per statistics block: at most kStatBlocks blocks, four waves each.
int stat_tpb(int T_) {
  const int tpb = (T_ + kStatBlocks - 1) / kStatBlocks;
  return std::max(4, (tpb + 3) / 4 * 4);
}

// ------------------------------------------------- balance loss -> router
// C[M, N] += A[M, K] B[K, N] with fp32 products summed in ascending k, for the
// router's share of a dense logit gradient dl [T, E] (logits = x W_r):
//   dx      = dl W_r^T : M = T, N = d, K = E; A = dl rows, B[k][n] = W_r[n][k];
//   dW_r^T  = dl^T x   : M = E, N = d, K = T; A[m][k] = dl[k][m], B = x rows.
// A block owns a 32 x 256 tile of C and walks K in 32-deep chunks staged in
// LDS as fp32 (the next chunk's global loads are in flight while the current
// one is summed); each thread keeps a 4 x 8 register tile.  DX: add the tile
// to dx in place (one rounding).  Otherwise (dW_r^T): the K range is split in
// blocks of kDenseChunk tokens (grid.z) whose fp32 partials go to part[z] and
// are summed in order by router_dense_wsum_kernel.
constexpr int kDenseChunk = 512;  // tokens per dW_r partial
template <typename T, bool DX>
__global__ void __launch_bounds__(256) router_dense_kernel(const float* __restrict__ dl,
                                                           const T* __restrict__ b, int T_, int d,
                                                           int E, T* __restrict__ dx,
                                                           float* __restrict__ part) {
  __shared__ float As[32][36];   // [k][m] (16-byte aligned rows)
  __shared__ float Bs[32][260];  // [k][n]
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int NQ = 32 / V;         // B vectors per thread per chunk
  const int tid = threadIdx.x;
  const int M = DX ? T_ : E;
  const int K = DX ? E : T_;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 256;
  const int kbeg = DX ? 0 : blockIdx.z * kDenseChunk;
  const int kend = DX ? K : min(K, kbeg + kDenseChunk);
  const int mg = tid >> 5, ng = tid & 31;  // 8 x 32 threads: C rows 4 mg.., columns 8 ng..
  const int ar = tid >> 3, ac = (tid & 7) * 4;  // A staging: row, first of 4 columns
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  float areg[4], breg[NQ][V];
  // global -> registers of the K chunk at k0 (zeros past the edges)
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // DX: A row m = ar, k = ac + q (dl rows); else A[m][k] = dl[k][m]: row k = ar
      const int m = DX ? m0 + ar : m0 + ac + q, k = DX ? k0 + ac + q : k0 + ar;
      areg[q] = (m < M && k < kend) ? dl[DX ? (size_t)m * E + k : (size_t)k * E + m] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int v = 0; v < V; ++v) breg[q][v] = 0.f;
      if (DX) {
        // B[k][n] = W_r[n][k]: V consecutive k of W_r row n = n0 + tid
        const int n = n0 + tid, kk = k0 + q * V;
        if (n < d) {
          const T* src = b + (size_t)n * E + kk;
          if (E % V == 0 && kk + V <= kend) {
            const uint4 raw = *reinterpret_cast<const uint4*>(src);
            const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int v = 0; v < V; ++v) breg[q][v] = Elem<T>::ld(e, v);
          } else {
#pragma unroll
            for (int v = 0; v < V; ++v)
              if (kk + v < kend) breg[q][v] = Elem<T>::ld(src, v);
          }
        }
      } else {
        // B = x rows: V consecutive n of row k
        const int idx = q * 256 + tid;
        const int r = idx / (256 / V), c = (idx % (256 / V)) * V;
        const int k = k0 + r, n = n0 + c;
        if (k < kend && n < d) {
          const uint4 raw = *reinterpret_cast<const uint4*>(b + (size_t)k * d + n);
          const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
          for (int v = 0; v < V; ++v) breg[q][v] = Elem<T>::ld(e, v);
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (DX) As[ac + q][ar] = areg[q];
      else As[ar][ac + q] = areg[q];
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (DX) {
#pragma unroll
        for (int v = 0; v < V; ++v) Bs[q * V + v][tid] = breg[q][v];
      } else {
        const int idx = q * 256 + tid;
        const int r = idx / (256 / V), c = (idx % (256 / V)) * V;
#pragma unroll
        for (int v = 0; v < V; ++v) Bs[r][c + v] = breg[q][v];
      }
    }
  };
  if (kbeg < kend) load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += 32) {
    __syncthreads();  // the previous chunk's sums are done with the tiles
    stash();
    __syncthreads();
    if (k0 + 32 < kend) load(k0 + 32);  // in flight while this chunk is summed
#pragma unroll 4
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], bv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][mg * 4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = Bs[kk][ng * 8 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], bv[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + mg * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + ng * 8 + j;
      if (n >= d) continue;
      if (DX) {
        const size_t o = (size_t)m * d + n;
        Elem<T>::st(dx, o, Elem<T>::ld(dx, o) + acc[i][j]);
      } else {
        part[((size_t)blockIdx.z * E + m) * d + n] = acc[i][j];
      }
    }
  }
}

// Inputs of the matrix-core path: dl rounded to bf16 (nearest even), W_r^T
// [E,d] from W_r [d,E], and the token-chunk offsets {0, 512, ..., T}.
__global__ void dense_prep_kernel(const float* __restrict__ dl, long long n_dl,
                                  const bf16_t* __restrict__ wr, int d, int E, int T_, int nz,
                                  bf16_t* __restrict__ dlb, bf16_t* __restrict__ wrt,
                                  int32_t* __restrict__ voff) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_dl; i += stride)
    dlb[i] = f2bf(dl[i]);
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < (long long)d * E; i += stride) {
    const int e = (int)(i / d), n = (int)(i % d);  // wrt[e][n] = wr[n][e]
    wrt[i] = wr[(size_t)n * E + e];
  }
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i <= nz; i += stride)
    voff[i] = (int32_t)min((long long)T_, i * kDenseChunk);
}

// dW_r[i][e] += sum over chunks z (in order) of part[z][i][e] (the matrix-core
// path's [d][E] partials), one rounding.
__global__ void __launch_bounds__(256) router_dense_sum_de_kernel(const float* __restrict__ part, int nz,
                                                                  long long n, bf16_t* __restrict__ dwr) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < nz; ++z) s += part[(size_t)z * n + i];
  dwr[i] = f2bf(bf2f(dwr[i]) + s);
}

// dW_r[n][e] += sum over chunks z (in order) of part[z][e][n], one rounding.
template <typename T>
__global__ void __launch_bounds__(256) router_dense_wsum_kernel(const float* __restrict__ part,
                                                                int nz, int d, int E,
                                                                T* __restrict__ dwr) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // e * d + n
  if (i >= (long long)E * d) return;
  const int e = (int)(i / d), n = (int)(i % d);
  float s = 0.f;
  for (int z = 0; z < nz; ++z) s += part[(size_t)z * E * d + i];
  const size_t o = (size_t)n * E + e;
  Elem<T>::st(dwr, o, Elem<T>::ld(dwr, o) + s);
}

}  // namespace

// ---------------------------------------------------------------- C ABI
using namespace moe_host;

// Workspace of moe_route_stats (three [E][256] partial arrays and the [E]
// loss terms) and of moe_expert_grad_norms ([E][256] partial sums); both fit
// in the larger.
// Workspace of moe_router_dense_bwd: fp32 dW_r partials, one [E, d] block per
// kDenseChunk tokens; the matrix-core path (bf16) also keeps dl in bf16, W_r^T
// and the chunk offsets in front of them.
static size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t moe_internal_router_dense_ws_bytes(int T_, int d, int E) {
  const size_t nz = (size_t)(T_ + kDenseChunk - 1) / kDenseChunk;
  return a256((size_t)T_ * E * 2) + a256((size_t)E * d * 2) + a256((nz + 1) * 4) +
         a256(nz * E * d * sizeof(float));
}

moe_status moe_internal_router_dense_mfma(moe_ctx* ctx, const bf16_t* x, const bf16_t* dlb,
                                          const bf16_t* wrt, const int32_t* voff, int nz, int T_,
                                          int d, int E, bf16_t* dx, float* part);  // gemm_bf16.hip

size_t moe_internal_stats_ws_bytes(int E) {
  const size_t a = (size_t)kStatBlocks * E * 12 + (size_t)E * 4, b = (size_t)E * kNormChunks * 4;
  return ((a > b ? a : b) + 255) & ~(size_t)255;
}

#define STATS_EPL_DISPATCH(E, CALL) \
  do {                              \
    if ((E) <= 64) {                \
      constexpr int EPL = 1;        \
      CALL;                         \
    } else if ((E) <= 128) {        \
      constexpr int EPL = 2;        \
      CALL;                         \
    } else if ((E) <= 256) {        \
      constexpr int EPL = 4;        \
      CALL;                         \
    } else if ((E) <= 512) {        \
      constexpr int EPL = 8;        \
      CALL;                         \
    } else {                        \
      constexpr int EPL = 16;       \
      CALL;                         \
    }                               \
  } while (0)

extern "C" {

moe_status moe_route_stats(moe_ctx* ctx, const float* logits, const int32_t* counts, int T_, int E,
                           int k, float alpha, float* prob_mean, int32_t* top1_count,
                           float* top1_prob_mean, float* aux_loss) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, T_ >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= E && k <= 32,
              "moe_route_stats: bad shape T=%d E=%d k=%d", T_, E, k);
  MOE_REQUIRE(ctx, std::isfinite(alpha), "moe_route_stats: alpha is not finite");
  MOE_REQUIRE(ctx, counts && prob_mean && top1_count && top1_prob_mean && aux_loss,
              "moe_route_stats: null output or counts");
  MOE_REQUIRE(ctx, T_ == 0 || logits, "moe_route_stats: logits is null");
  MOE_REQUIRE_DISJOINT(ctx, "moe_route_stats", {prob_mean, (size_t)E * 4, "prob_mean"},
                       {top1_count, (size_t)E * 4, "top1_count"},
                       {top1_prob_mean, (size_t)E * 4, "top1_prob_mean"}, {aux_loss, 4, "aux_loss"});
  const size_t need = moe_internal_stats_ws_bytes(E);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "moe_route_stats: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  const int tpb = stat_tpb(T_);
  const int nblk = T_ > 0 ? (T_ + tpb - 1) / tpb : 0;
  float* part_p = (float*)ctx->ws;
  float* part_s = part_p + (size_t)kStatBlocks * E;
  int32_t* part_c = (int32_t*)(part_s + (size_t)kStatBlocks * E);
  float* term = (float*)(part_c + (size_t)kStatBlocks * E);
  const double scale = (double)alpha * E / ((double)std::max(T_, 1) * k);
  moe_prof_scope ps(ctx, MOE_K_ROUTE_STATS);
  if (nblk > 0)
    STATS_EPL_DISPATCH(E, (stats_partial_kernel<EPL><<<nblk, 256, 0, ctx->stream>>>(
                               logits, T_, E, tpb, part_p, part_s, part_c)));
  stats_expert_kernel<<<(E + 3) / 4, 256, 0, ctx->stream>>>(part_p, part_s, part_c, nblk, counts, T_, E,
                                                            prob_mean, top1_count, top1_prob_mean, term);
  stats_loss_kernel<<<1, 1024, 0, ctx->stream>>>(term, E, (float)scale, aux_loss);
  return check_launch(ctx, "moe_route_stats");
}

moe_status moe_aux_loss_bwd(moe_ctx* ctx, const float* logits, const int32_t* counts, int T_, int E,
                            int k, float alpha, float dloss, float* dlogits) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, T_ >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= E && k <= 32,
              "moe_aux_loss_bwd: bad shape T=%d E=%d k=%d", T_, E, k);
  MOE_REQUIRE(ctx, std::isfinite(alpha) && std::isfinite(dloss), "moe_aux_loss_bwd: alpha or dloss not finite");
  if (T_ == 0) return MOE_OK;
  MOE_REQUIRE(ctx, logits && counts && dlogits, "moe_aux_loss_bwd: null pointer");
  const double coef = (double)dloss * alpha * E / ((double)T_ * T_ * k);
  const int blocks = std::min(2048, (T_ + 15) / 16);
  moe_prof_scope ps(ctx, MOE_K_AUX_BWD);
  STATS_EPL_DISPATCH(E, (aux_bwd_kernel<EPL><<<blocks, 256, 0, ctx->stream>>>(logits, counts, T_, E,
                                                                               (float)coef, dlogits)));
  return check_launch(ctx, "moe_aux_loss_bwd");
}

moe_status moe_router_dense_bwd(moe_ctx* ctx, const void* x, const void* w_router,
                                const float* dlogits, int T_, int d, int E, moe_dtype dtype,
                                void* dx, void* dw_router) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE_DTYPE(ctx, dtype);
  MOE_REQUIRE(ctx, T_ >= 0 && T_ <= 65535 * 32 && d >= 8 && d % 8 == 0 && E >= 1 && E <= 1024,
              "moe_router_dense_bwd: bad shape T=%d d=%d E=%d", T_, d, E);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, x, T_ == 0);
  MOE_REQUIRE_PTR(ctx, w_router);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dlogits, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dx, T_ == 0);
  MOE_REQUIRE_PTR(ctx, dw_router);
  MOE_REQUIRE_DISJOINT(ctx, "moe_router_dense_bwd", {dx, (size_t)T_ * d * esize(dtype), "dx"},
                       {dw_router, (size_t)d * E * esize(dtype), "dw_router"});
  if (T_ == 0) return MOE_OK;  // nothing to add
  const size_t need = moe_internal_router_dense_ws_bytes(T_, d, E);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "moe_router_dense_bwd: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  float* part = (float*)ctx->ws;
  const int nz = (T_ + kDenseChunk - 1) / kDenseChunk;
  const dim3 gdx((d + 255) / 256, (T_ + 31) / 32), gdw((d + 255) / 256, (E + 31) / 32, nz);
  const unsigned gsum = (unsigned)(((long long)E * d + 255) / 256);
  moe_prof_scope ps(ctx, MOE_K_ROUTER_DENSE_BWD);
  if (dtype == MOE_BF16 && d % 64 == 0 && E % 64 == 0) {
    // matrix cores: dl rounded to bf16 as the GEMM operand, fp32 sums
    char* w = (char*)ctx->ws;
    bf16_t* dlb = (bf16_t*)w;
    w += a256((size_t)T_ * E * 2);
    bf16_t* wrt = (bf16_t*)w;
    w += a256((size_t)E * d * 2);
    int32_t* voff = (int32_t*)w;
    w += a256((size_t)(nz + 1) * 4);
    float* pde = (float*)w;
    dense_prep_kernel<<<1024, 256, 0, ctx->stream>>>(dlogits, (long long)T_ * E, (const bf16_t*)w_router,
                                                     d, E, T_, nz, dlb, wrt, voff);
    moe_status st = moe_internal_router_dense_mfma(ctx, (const bf16_t*)x, dlb, wrt, voff, nz, T_, d, E,
                                                   (bf16_t*)dx, pde);
    if (st != MOE_OK) return st;
    router_dense_sum_de_kernel<<<gsum, 256, 0, ctx->stream>>>(pde, nz, (long long)d * E, (bf16_t*)dw_router);
  } else if (dtype == MOE_BF16) {
    router_dense_kernel<bf16_t, true><<<gdx, 256, 0, ctx->stream>>>(
        dlogits, (const bf16_t*)w_router, T_, d, E, (bf16_t*)dx, nullptr);
    router_dense_kernel<bf16_t, false><<<gdw, 256, 0, ctx->stream>>>(
        dlogits, (const bf16_t*)x, T_, d, E, nullptr, part);
    router_dense_wsum_kernel<bf16_t><<<gsum, 256, 0, ctx->stream>>>(part, nz, d, E, (bf16_t*)dw_router);
  } else {
    router_dense_kernel<float, true><<<gdx, 256, 0, ctx->stream>>>(
        dlogits, (const float*)w_router, T_, d, E, (float*)dx, nullptr);
    router_dense_kernel<float, false><<<gdw, 256, 0, ctx->stream>>>(
        dlogits, (const float*)x, T_, d, E, nullptr, part);
    router_dense_wsum_kernel<float><<<gsum, 256, 0, ctx->stream>>>(part, nz, d, E, (float*)dw_router);
  }
  return check_launch(ctx, "moe_router_dense_bwd");
}

moe_status moe_expert_grad_norms(moe_ctx* ctx, const void* dw, int E, int rows, int cols,
                                 moe_dtype dtype, float* norms) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE_DTYPE(ctx, dtype);
  const int vec = dtype == MOE_F32 ? 4 : 8;
  MOE_REQUIRE(ctx, E >= 1 && E <= 1024 && rows >= 0 && cols >= 0 && cols % vec == 0 &&
                       (long long)rows * cols < (1LL << 40),
              "moe_expert_grad_norms: bad shape E=%d rows=%d cols=%d (cols %% %d == 0)", E, rows,
              cols, vec);
  MOE_REQUIRE(ctx, norms != nullptr, "moe_expert_grad_norms: norms is null");
  const size_t n = (size_t)rows * cols;
  MOE_REQUIRE(ctx, n == 0 || (dw && aligned16(dw)), "moe_expert_grad_norms: dw null or not 16-byte aligned");
  const size_t need = moe_internal_stats_ws_bytes(E);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "moe_expert_grad_norms: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  // chunks per expert: enough blocks to cover the chip, each a whole number
  // of 16-byte vectors of one expert
  const size_t nvec = n / vec;
  int nchunk = std::min<int>(kNormChunks, std::max(1, (2048 + E - 1) / E));
  nchunk = (int)std::max<size_t>(1, std::min<size_t>(nchunk, nvec));
  const size_t per = (nvec + nchunk - 1) / nchunk * vec;
  float* part = (float*)ctx->ws;
  moe_prof_scope ps(ctx, MOE_K_GRAD_NORMS);
  if (n > 0) {
    dim3 grid(nchunk, E);
    if (dtype == MOE_F32)
      grad_norm_partial_kernel<float><<<grid, 256, 0, ctx->stream>>>((const float*)dw, n, per, part);
    else
      grad_norm_partial_kernel<bf16_t><<<grid, 256, 0, ctx->stream>>>((const bf16_t*)dw, n, per, part);
  } else {
    nchunk = 0;
  }
  grad_norm_final_kernel<<<(E + 255) / 256, 256, 0, ctx->stream>>>(part, nchunk, E, norms);
  return check_launch(ctx, "moe_expert_grad_norms");
}

}  // extern "C"
