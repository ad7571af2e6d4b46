// rows.hip — row movement: rowwise permute into the expert buffers, the
// gate-weighted unpermute-combine, and their backward passes.
//
// Pages: routed rows are written straight into the experts' input buffers
// ([P1] 核心特点 二, rowwise expert parallelism); results return along the
// original path and are restored to token order ([P2] 2.1); the backward moves
// every token again ([P2] 1.2).
//
// All four kernels are HBM-bound row copies: one wave owns one token at a time
// and moves its rows in 16-byte lane chunks (1 KiB per wave instruction), so
// every global access is a fully coalesced 16-byte vector access.  The k row
// indices of the token are wave-uniform scalar loads.
//
// Cache policy (measured on the whole layer): every row the combine backward
// and the permute backward read or write goes nontemporal.  The dyp rows the
// down dgrad reads next then reach HBM during the row kernel instead of
// sitting dirty in L2 while the GEMM streams its operands (down dgrad about
// 2 % faster, the combine backward itself 6 % faster), and rows read once do
// not evict GEMM operands.  The combine keeps cached loads (the combine
// backward re-reads the same expert outputs).  The permute keeps cached
// stores: nontemporal ones speed the gate/up GEMM after it by about as much
// as they slow the permute.
#include <hip/hip_runtime.h>

#include "common.h"

using namespace moe;

namespace {

// 16-byte nontemporal load and store.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
__device__ __forceinline__ uint4 ntld(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void ntst(uint4 v, uint4* p) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4_t*)p);
}

template <typename T>
struct Vec {
  static constexpr int N = 16 / sizeof(T);
};

__device__ __forceinline__ void unpack(const uint4& r, float (&f)[8], bf16_t) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const uint4& r, float (&f)[4], float) {
  f[0] = __uint_as_float(r.x);
  f[1] = __uint_as_float(r.y);
  f[2] = __uint_as_float(r.z);
  f[3] = __uint_as_float(r.w);
}
__device__ __forceinline__ uint4 pack(const float (&f)[8], bf16_t) {
  return make_uint4(pack2bf(f[0], f[1]), pack2bf(f[2], f[3]), pack2bf(f[4], f[5]),
                    pack2bf(f[6], f[7]));
}
__device__ __forceinline__ uint4 pack(const float (&f)[4], float) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}

constexpr int kWaves = 4;  // waves per block; one token per wave at a time
// Chunks per lane loaded before any is used: every gather of a token (CPL
// chunks of each of its k rows) is in flight at once.
template <int KMAX>
constexpr int chunks_per_lane() { return KMAX >= 16 ? 1 : 16 / KMAX; }
constexpr int kPermuteCPL = 8;
template <int KMAX, bool ROUTER>
constexpr int permute_bwd_cpl() { return ROUTER ? (KMAX >= 8 ? 1 : 8 / KMAX) : chunks_per_lane<KMAX>(); }

// FULL (every kernel below): the token has exactly KMAX rows and its row is a
// whole number of lane passes (nchunk a multiple of 64 * CPL).  The loads then
// carry no guard, so all of a token's loads issue back to back; with the
// guards each load sat behind a branch and a wait for the one before
// (permute backward 67 -> 59 us at 16384 tokens x 2048 bf16, top-4, with the
// caches holding no rows; the combine 62 -> 61 us).

// xp[row_of[t,j]] = x[t]: read each token row once, write its k copies.
template <int KMAX, bool FULL>
__global__ void __launch_bounds__(256) permute_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ row_of, int T_,
                                                      int nchunk, int k_arg, uint4* __restrict__ xp) {
  constexpr int CPL = kPermuteCPL;
  const int k = FULL ? KMAX : k_arg;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  for (int t = wave; t < T_; t += nw) {
    int rows[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) rows[j] = j < k ? row_of[(size_t)t * k + j] : 0;
    const uint4* src = x + (size_t)t * nchunk;
    for (int cb = lane; cb < nchunk; cb += 64 * CPL) {
      uint4 v[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        v[u] = FULL || cb + 64 * u < nchunk ? src[cb + 64 * u] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = cb + 64 * u;
        if (FULL || c < nchunk) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j)
            if (j < k) xp[(size_t)rows[j] * nchunk + c] = v[u];
        }
      }
    }
  }
}

// y[t] = sum_j gates[t,j] * yp[row_of[t,j]] (+ add[t], the shared expert's
// row, when add is given), slot order then the addend, fp32 sums.
template <typename T, int KMAX, bool FULL>
__global__ void __launch_bounds__(256) combine_kernel(const uint4* __restrict__ yp,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ row_of, int T_,
                                                      int nchunk, int k_arg, const uint4* __restrict__ add,
                                                      uint4* __restrict__ y) {
  constexpr int V = Vec<T>::N;
  constexpr int CPL = chunks_per_lane<KMAX>();
  const int k = FULL ? KMAX : k_arg;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  for (int t = wave; t < T_; t += nw) {
    int rows[KMAX];
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? row_of[(size_t)t * k + j] : 0;
      g[j] = j < k ? gates[(size_t)t * k + j] : 0.f;
    }
    for (int cb = lane; cb < nchunk; cb += 64 * CPL) {
      uint4 raw[CPL][KMAX];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k && (FULL || cb + 64 * u < nchunk)) raw[u][j] = yp[(size_t)rows[j] * nchunk + cb + 64 * u];
      __builtin_amdgcn_sched_barrier(0);  // every load above issues before the first use
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = cb + 64 * u;
        if (!FULL && c >= nchunk) continue;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < k) {
            float f[V];
            unpack(raw[u][j], f, T());
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] += g[j] * f[i];
          }
        }
        if (add) {
          float f[V];
          unpack(add[(size_t)t * nchunk + c], f, T());
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += f[i];
        }
        y[(size_t)t * nchunk + c] = pack(acc, T());
      }
    }
  }
}

// dyp[row_of[t,j]] = gates[t,j] * dy[t];  dgates[t,j] = <dy[t], yp[row_of[t,j]]>.
// The dot products are lane partials (chunk order) reduced across the wave in
// a fixed order.
template <typename T, int KMAX, bool FULL>
__global__ void __launch_bounds__(256) combine_bwd_kernel(
    const uint4* __restrict__ dy, const uint4* __restrict__ yp, const float* __restrict__ gates,
    const int32_t* __restrict__ row_of, int T_, int nchunk, int k_arg, uint4* __restrict__ dyp,
    float* __restrict__ dgates) {
  constexpr int V = Vec<T>::N;
  constexpr int CPL = chunks_per_lane<KMAX>();
  const int k = FULL ? KMAX : k_arg;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  for (int t = wave; t < T_; t += nw) {
    int rows[KMAX];
    float g[KMAX], dot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? row_of[(size_t)t * k + j] : 0;
      g[j] = j < k ? gates[(size_t)t * k + j] : 0.f;
      dot[j] = 0.f;
    }
    for (int cb = lane; cb < nchunk; cb += 64 * CPL) {
      uint4 draw[CPL], raw[CPL][KMAX];
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = cb + 64 * u;
        if (FULL || c < nchunk) {
          draw[u] = ntld(&dy[(size_t)t * nchunk + c]);
#pragma unroll
          for (int j = 0; j < KMAX; ++j)
            if (j < k) raw[u][j] = ntld(&yp[(size_t)rows[j] * nchunk + c]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // every load above issues before the first use
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = cb + 64 * u;
        if (!FULL && c >= nchunk) continue;
        float d[V];
        unpack(draw[u], d, T());
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < k) {
            float f[V], o[V];
            unpack(raw[u][j], f, T());
#pragma unroll
            for (int i = 0; i < V; ++i) {
              dot[j] += d[i] * f[i];
              o[i] = g[j] * d[i];
            }
            ntst(pack(o, T()), &dyp[(size_t)rows[j] * nchunk + c]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      float v = dot[j];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      dot[j] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) dgates[(size_t)t * k + j] = dot[j];
    }
  }
}

// dx[t] = sum_j dxp[row_of[t,j]] (+ add[t], the shared expert's input
// gradient, when add is given) + sum_j dl[t,j] * W_r^T[topk[t,j]] (router
// term optional; W_r^T is [E,d], made by transpose_kernel), in that order.
template <typename T, int KMAX, bool ROUTER, bool FULL>
__global__ void __launch_bounds__(256) permute_bwd_kernel(
    const uint4* __restrict__ dxp, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ topk, const float* __restrict__ dls,
    const uint4* __restrict__ wrt, int T_, int nchunk, int k_arg, const uint4* __restrict__ add,
    uint4* __restrict__ dx) {
  constexpr int V = Vec<T>::N;
  const int k = FULL ? KMAX : k_arg;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  for (int t = wave; t < T_; t += nw) {
    int rows[KMAX], ex[KMAX];
    float w[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? row_of[(size_t)t * k + j] : 0;
      if (ROUTER) {
        ex[j] = j < k ? topk[(size_t)t * k + j] : 0;
        w[j] = j < k ? dls[(size_t)t * k + j] : 0.f;
      }
    }
    constexpr int CPL = permute_bwd_cpl<KMAX, ROUTER>();
    for (int cb = lane; cb < nchunk; cb += 64 * CPL) {
      uint4 raw[CPL][KMAX], wraw[CPL][ROUTER ? KMAX : 1];
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = cb + 64 * u;
        if (FULL || c < nchunk) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
              raw[u][j] = ntld(&dxp[(size_t)rows[j] * nchunk + c]);
              if (ROUTER) wraw[u][ROUTER ? j : 0] = wrt[(size_t)ex[j] * nchunk + c];
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // every load above issues before the first use
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = cb + 64 * u;
        if (!FULL && c >= nchunk) continue;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < k) {
            float f[V];
            unpack(raw[u][j], f, T());
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] += f[i];
          }
        }
        if (add) {
          float f[V];
          unpack(add[(size_t)t * nchunk + c], f, T());
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += f[i];
        }
        if (ROUTER) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
              float f[V];
              unpack(wraw[u][ROUTER ? j : 0], f, T());
#pragma unroll
              for (int i = 0; i < V; ++i) acc[i] += w[j] * f[i];
            }
          }
        }
        ntst(pack(acc, T()), &dx[(size_t)t * nchunk + c]);
      }
    }
  }
}

// out[e][i] = in[i][e] for a [d,E] matrix (router weights, small).
template <typename T>
__global__ void transpose_kernel(const T* __restrict__ in, int d, int E, T* __restrict__ out) {
  __shared__ T tile[32][33];
  const int i0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: 8 rows at a time
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, e = e0 + tx;
    if (i < d && e < E) tile[r][tx] = in[(size_t)i * E + e];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, i = i0 + tx;
    if (i < d && e < E) out[(size_t)e * d + i] = tile[tx][r];
  }
}

int grid_for(int T_) {
  const int want = (T_ + kWaves - 1) / kWaves;
  return want < 8192 ? (want > 0 ? want : 1) : 8192;
}

}  // namespace

// ---------------------------------------------------------------- C ABI
using namespace moe_host;

size_t moe_internal_wrt_bytes(int d, int E, moe_dtype dt);

#define ROWS_DISPATCH_K(KVAR, LAUNCH) \
  do {                                \
    if (KVAR <= 2) {                  \
      constexpr int KM = 2;           \
      LAUNCH;                         \
    } else if (KVAR <= 4) {           \
      constexpr int KM = 4;           \
      LAUNCH;                         \
    } else if (KVAR <= 8) {           \
      constexpr int KM = 8;           \
      LAUNCH;                         \
    } else {                          \
      constexpr int KM = 32;          \
      LAUNCH;                         \
    }                                 \
  } while (0)

// Launches LAUNCH with FULL = COND (a compile-time constant inside it).
#define ROWS_FULL(COND, LAUNCH)       \
  do {                                \
    if (COND) {                       \
      constexpr bool FULL = true;     \
      LAUNCH;                         \
    } else {                          \
      constexpr bool FULL = false;    \
      LAUNCH;                         \
    }                                 \
  } while (0)

static moe_status rows_common(moe_ctx* ctx, int T_, int d, int k, moe_dtype dtype,
                              const char* what) {
  MOE_REQUIRE_DTYPE(ctx, dtype);
  MOE_REQUIRE(ctx, T_ >= 0 && d >= 8 && d % 8 == 0 && k >= 1 && k <= 32,
              "%s: bad shape T=%d d=%d k=%d", what, T_, d, k);
  MOE_REQUIRE(ctx, (int64_t)T_ * k < (int64_t)1 << 31, "%s: T*k >= 2^31", what);
  return MOE_OK;
}

extern "C" {

moe_status moe_permute(moe_ctx* ctx, const void* x, const int32_t* row_of, int T_, int d, int k,
                       moe_dtype dtype, void* xp) {
  MOE_CHECK_CTX(ctx);
  moe_status st = rows_common(ctx, T_, d, k, dtype, "moe_permute");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, x, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, row_of, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, xp, T_ == 0);
  if (T_ == 0) return MOE_OK;
  const int nchunk = (int)(d * esize(dtype) / 16);
  moe_prof_scope ps(ctx, MOE_K_PERMUTE);
  ROWS_DISPATCH_K(k, ROWS_FULL(k == KM && nchunk % (64 * kPermuteCPL) == 0,
                               (permute_kernel<KM, FULL><<<grid_for(T_), 256, 0, ctx->stream>>>(
                                   (const uint4*)x, row_of, T_, nchunk, k, (uint4*)xp))));
  return check_launch(ctx, "moe_permute");
}

}  // extern "C"

static moe_status combine_impl(moe_ctx* ctx, const void* yp, const float* gates,
                               const int32_t* row_of, const void* add, int T_, int d, int k,
                               moe_dtype dtype, void* y) {
  MOE_CHECK_CTX(ctx);
  moe_status st = rows_common(ctx, T_, d, k, dtype, "moe_combine");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, yp, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, gates, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, row_of, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, y, T_ == 0);
  if (T_ == 0) return MOE_OK;
  const int nchunk = (int)(d * esize(dtype) / 16);
  moe_prof_scope ps(ctx, MOE_K_COMBINE);
#define CB_LAUNCH(TY)                                                                          \
  ROWS_DISPATCH_K(k, ROWS_FULL(k == KM && nchunk % (64 * chunks_per_lane<KM>()) == 0,           \
                               (combine_kernel<TY, KM, FULL><<<grid_for(T_), 256, 0, ctx->stream>>>( \
                                   (const uint4*)yp, gates, row_of, T_, nchunk, k,            \
                                   (const uint4*)add, (uint4*)y))))
  if (dtype == MOE_BF16)
    CB_LAUNCH(bf16_t);
  else
    CB_LAUNCH(float);
#undef CB_LAUNCH
  return check_launch(ctx, "moe_combine");
}

extern "C" {

moe_status moe_combine(moe_ctx* ctx, const void* yp, const float* gates, const int32_t* row_of,
                       int T_, int d, int k, moe_dtype dtype, void* y) {
  return combine_impl(ctx, yp, gates, row_of, nullptr, T_, d, k, dtype, y);
}

moe_status moe_combine_shared(moe_ctx* ctx, const void* yp, const float* gates,
                              const int32_t* row_of, const void* y_shared, int T_, int d, int k,
                              moe_dtype dtype, void* y) {
  MOE_REQUIRE(ctx, ctx == nullptr || T_ == 0 || (y_shared && aligned16(y_shared)),
              "moe_combine_shared: y_shared null or not 16-byte aligned");
  return combine_impl(ctx, yp, gates, row_of, y_shared, T_, d, k, dtype, y);
}

moe_status moe_combine_bwd(moe_ctx* ctx, const void* dy, const void* yp, const float* gates,
                           const int32_t* row_of, int T_, int d, int k, moe_dtype dtype,
                           void* dyp, float* dgates) {
  MOE_CHECK_CTX(ctx);
  moe_status st = rows_common(ctx, T_, d, k, dtype, "moe_combine_bwd");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dy, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, yp, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, gates, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, row_of, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dyp, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dgates, T_ == 0);
  MOE_REQUIRE_DISJOINT(ctx, "moe_combine_bwd", {dyp, (size_t)T_ * k * d * esize(dtype), "dyp"},
                       {dgates, (size_t)T_ * k * 4, "dgates"});
  if (T_ == 0) return MOE_OK;
  const int nchunk = (int)(d * esize(dtype) / 16);
  moe_prof_scope ps(ctx, MOE_K_COMBINE_BWD);
#define CBB_LAUNCH(TY)                                                                         \
  ROWS_DISPATCH_K(k, ROWS_FULL(k == KM && nchunk % (64 * chunks_per_lane<KM>()) == 0,           \
                               (combine_bwd_kernel<TY, KM, FULL><<<grid_for(T_), 256, 0, ctx->stream>>>( \
                                   (const uint4*)dy, (const uint4*)yp, gates, row_of, T_,     \
                                   nchunk, k, (uint4*)dyp, dgates))))
  if (dtype == MOE_BF16)
    CBB_LAUNCH(bf16_t);
  else
    CBB_LAUNCH(float);
#undef CBB_LAUNCH
  return check_launch(ctx, "moe_combine_bwd");
}

}  // extern "C"

static moe_status permute_bwd_impl(moe_ctx* ctx, const void* dxp, const int32_t* row_of,
                                   const int32_t* topk_idx, const float* dlogits_sel,
                                   const void* w_router, const void* add, int T_, int d, int E,
                                   int k, moe_dtype dtype, void* dx) {
  MOE_CHECK_CTX(ctx);
  moe_status st = rows_common(ctx, T_, d, k, dtype, "moe_permute_bwd");
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dxp, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, row_of, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dx, T_ == 0);
  const bool router = dlogits_sel != nullptr && w_router != nullptr;
  if (router) {
    MOE_REQUIRE(ctx, E >= 1 && E <= 1024 && k <= E, "moe_permute_bwd: bad E=%d", E);
    MOE_REQUIRE_PTR_OR_EMPTY(ctx, topk_idx, T_ == 0);
    MOE_REQUIRE_PTR(ctx, dlogits_sel);
    MOE_REQUIRE_PTR(ctx, w_router);
    const size_t need = moe_internal_wrt_bytes(d, E, dtype);
    if (ctx->ws == nullptr || ctx->ws_bytes < need)
      return fail(ctx, MOE_ERR_WORKSPACE, "moe_permute_bwd: workspace %zu bytes < %zu needed",
                  ctx->ws_bytes, need);
  }
  if (T_ == 0) return MOE_OK;
  const int nchunk = (int)(d * esize(dtype) / 16);
  moe_prof_scope ps(ctx, MOE_K_PERMUTE_BWD);
  if (router) {
    dim3 tg((d + 31) / 32, (E + 31) / 32);
    if (dtype == MOE_BF16)
      transpose_kernel<bf16_t><<<tg, 256, 0, ctx->stream>>>((const bf16_t*)w_router, d, E,
                                                            (bf16_t*)ctx->ws);
    else
      transpose_kernel<float><<<tg, 256, 0, ctx->stream>>>((const float*)w_router, d, E,
                                                           (float*)ctx->ws);
  }
  const uint4* wrt = (const uint4*)ctx->ws;
#define PB_LAUNCH(TY)                                                                          \
  do {                                                                                         \
    if (router)                                                                                \
      ROWS_DISPATCH_K(k, ROWS_FULL(k == KM && nchunk % (64 * permute_bwd_cpl<KM, true>()) == 0, \
          (permute_bwd_kernel<TY, KM, true, FULL><<<grid_for(T_), 256, 0, ctx->stream>>>(      \
              (const uint4*)dxp, row_of, topk_idx, dlogits_sel, wrt, T_, nchunk, k,            \
              (const uint4*)add, (uint4*)dx))));                                               \
    else                                                                                       \
      ROWS_DISPATCH_K(k, ROWS_FULL(k == KM && nchunk % (64 * permute_bwd_cpl<KM, false>()) == 0, \
          (permute_bwd_kernel<TY, KM, false, FULL><<<grid_for(T_), 256, 0, ctx->stream>>>(     \
              (const uint4*)dxp, row_of, nullptr, nullptr, nullptr, T_, nchunk, k,             \
              (const uint4*)add, (uint4*)dx))));                                               \
  } while (0)
  if (dtype == MOE_BF16)
    PB_LAUNCH(bf16_t);
  else
    PB_LAUNCH(float);
#undef PB_LAUNCH
  return check_launch(ctx, "moe_permute_bwd");
}

extern "C" {

moe_status moe_permute_bwd(moe_ctx* ctx, const void* dxp, const int32_t* row_of,
                           const int32_t* topk_idx, const float* dlogits_sel,
                           const void* w_router, int T_, int d, int E, int k, moe_dtype dtype,
                           void* dx) {
  return permute_bwd_impl(ctx, dxp, row_of, topk_idx, dlogits_sel, w_router, nullptr, T_, d, E, k,
                          dtype, dx);
}

moe_status moe_permute_bwd_shared(moe_ctx* ctx, const void* dxp, const int32_t* row_of,
                                  const int32_t* topk_idx, const float* dlogits_sel,
                                  const void* w_router, const void* dx_shared, int T_, int d, int E,
                                  int k, moe_dtype dtype, void* dx) {
  MOE_REQUIRE(ctx, ctx == nullptr || T_ == 0 || (dx_shared && aligned16(dx_shared)),
              "moe_permute_bwd_shared: dx_shared null or not 16-byte aligned");
  return permute_bwd_impl(ctx, dxp, row_of, topk_idx, dlogits_sel, w_router, dx_shared, T_, d, E,
                          k, dtype, dx);
}

}  // extern "C"
