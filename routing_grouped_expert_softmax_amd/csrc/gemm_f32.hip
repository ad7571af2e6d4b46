// gemm_f32.hip — fp32 grouped GEMMs for the SwiGLU experts (MOE_F32 data).
//
// Same operations, epilogues and device-side scheduling rules as the bf16
// matrix-core path, on the vector ALUs in fp32 (gfx950 has no fp32/xf32 MFMA
// rate worth a separate tile design for the small fp32 workload): 64x64 block
// tiles, BK = 16, each of the 256 threads computes a 4x4 block of outputs from
// LDS.  For the grouped-GEMM structure see gemm_bf16.hip.
#include <hip/hip_runtime.h>

#include "common.h"

using namespace moe;

namespace {

enum Mode : int { FWD_UP, FWD_DOWN, DGRAD_DOWN, DGRAD_UP, WGRAD_UP, WGRAD_DOWN };

struct P32 {
  const float* a0;
  const float* a1;
  int lda;
  const float* b0;
  const float* b1;
  int ldb;
  long long b_gstride;
  float* c0;
  float* c1;
  float* c2;
  int ldc;
  long long c_gstride;
  const float* aux0;
  const float* aux1;
  const int32_t* offsets;
  int E, M, N, K, kseg, ntiles, mtiles;
};

constexpr int T64 = 64, TK = 16;

template <int MODE>
__global__ void __launch_bounds__(256) gemm_f32_kernel(P32 p) {
  constexpr bool KRAG = (MODE == WGRAD_UP || MODE == WGRAD_DOWN);
  constexpr bool DUAL = (MODE == FWD_UP || MODE == WGRAD_UP);
  constexpr bool BKC = (MODE == DGRAD_DOWN || MODE == DGRAD_UP);  // B stored [n][k]
  __shared__ float As[TK][T64 + 1];
  __shared__ float Bs[2][TK][T64 + 1];
  __shared__ int info[3];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  int e, row0, rows, m0, nt;
  if (KRAG) {
    const int L = blockIdx.x;
    const int per_e = p.ntiles * p.mtiles;
    e = L / per_e;
    if (e >= p.E) return;
    nt = (L % per_e) / p.mtiles;
    m0 = ((L % per_e) % p.mtiles) * T64;
    row0 = p.offsets[e];
    rows = p.offsets[e + 1] - row0;
  } else {
    // serial search by one thread (the fp32 path serves small problems)
    if (tid == 0) {
      int L = blockIdx.x, found = -1, mt = 0, ntl = 0;
      for (int q = 0; q < p.E; ++q) {
        const int c = p.offsets[q + 1] - p.offsets[q];
        const int mt_q = (c + T64 - 1) / T64;
        const int til = mt_q * p.ntiles;
        if (L < til) {
          found = q;
          mt = L % mt_q;
          ntl = L / mt_q;
          break;
        }
        L -= til;
      }
      info[0] = found;
      info[1] = mt;
      info[2] = ntl;
    }
    __syncthreads();
    e = info[0];
    if (e < 0) return;
    nt = info[2];
    row0 = p.offsets[e] + info[1] * T64;
    rows = min(T64, p.offsets[e + 1] - row0);
    m0 = 0;
  }
  const float* bb0 = p.b0 + (size_t)e * p.b_gstride;
  const float* bb1 = p.b1 ? p.b1 + (size_t)e * p.b_gstride : nullptr;
  const int Klen = KRAG ? rows : p.K;
  float acc[2][4][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[s][i][j] = 0.f;

  for (int k0 = 0; k0 < Klen; k0 += TK) {
    // A tile: As[kk][mm] = A(m, k)
    for (int q = tid; q < TK * T64; q += 256) {
      const int kk = q / T64, mm = q % T64;
      const int k = k0 + kk;
      float v = 0.f;
      if (KRAG) {
        if (k < Klen && m0 + mm < p.M) v = p.a0[(size_t)(row0 + k) * p.lda + m0 + mm];
      } else if (mm < rows && k < Klen) {
        const float* a = p.a0;
        int kx = k;
        if (MODE == DGRAD_UP && k >= p.kseg) {
          a = p.a1;
          kx = k - p.kseg;
        }
        v = a[(size_t)(row0 + mm) * p.lda + kx];
      }
      As[kk][mm] = v;
    }
    // B tiles: Bs[s][kk][nn] = B_s(k, n)
    for (int s = 0; s < (DUAL ? 2 : 1); ++s) {
      for (int q = tid; q < TK * T64; q += 256) {
        const int kk = q / T64, nn = q % T64;
        const int k = k0 + kk, n = nt * T64 + nn;
        float v = 0.f;
        if (k < Klen && n < p.N) {
          const float* b = s ? bb1 : bb0;
          if (BKC) {
            int kx = k;
            if (MODE == DGRAD_UP && k >= p.kseg) {
              b = bb1;
              kx = k - p.kseg;
            }
            v = b[(size_t)n * p.ldb + kx];
          } else {
            const size_t krow = KRAG ? (size_t)(row0 + k) : (size_t)k;
            v = b[krow * p.ldb + n];
          }
        }
        Bs[s][kk][nn] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs[0][kk][tx * 4 + j];
        b1[j] = DUAL ? Bs[1][kk][tx * 4 + j] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[0][i][j] += a[i] * b0[j];
          if (DUAL) acc[1][i][j] += a[i] * b1[j];
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ml = ty * 4 + i;
    size_t crow;
    if (KRAG) {
      if (m0 + ml >= p.M) continue;
      crow = (size_t)(m0 + ml);
    } else {
      if (ml >= rows) continue;
      crow = (size_t)(row0 + ml);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nt * T64 + tx * 4 + j;
      if (n >= p.N) continue;
      size_t off = crow * p.ldc + n;
      if (KRAG) off += (size_t)e * p.c_gstride;
      const float v0 = acc[0][i][j], v1 = acc[1][i][j];
      if (MODE == FWD_UP) {
        p.c0[off] = v0;
        p.c1[off] = v1;
        p.c2[off] = v0 / (1.0f + expf(-v0)) * v1;
      } else if (MODE == DGRAD_DOWN) {
        const float g = p.aux0[off], u = p.aux1[off];
        const float s = 1.0f / (1.0f + expf(-g));
        p.c0[off] = v0 * u * s * (1.0f + g * (1.0f - s));
        p.c1[off] = v0 * g * s;
      } else if (MODE == WGRAD_UP) {
        p.c0[off] = v0;
        p.c1[off] = v1;
      } else {
        p.c0[off] = v0;
      }
    }
  }
}

template <int MODE>
hipError_t run(const P32& p, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  gemm_f32_kernel<MODE><<<blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

using namespace moe_host;

moe_status moe_internal_ffn_fwd_f32(moe_ctx* ctx, const float* xp, const float* wg,
                                    const float* wu, const float* wd, const int32_t* offsets,
                                    int E, int R, int d, int F, float* g, float* u, float* h,
                                    float* yp) {
  P32 p{};
  p.a0 = xp; p.lda = d;
  p.b0 = wg; p.b1 = wu; p.ldb = F; p.b_gstride = (long long)d * F;
  p.c0 = g; p.c1 = u; p.c2 = h; p.ldc = F;
  p.offsets = offsets; p.E = E; p.N = F; p.K = d; p.kseg = d;
  p.ntiles = (F + T64 - 1) / T64;
  hipError_t e = run<FWD_UP>(p, (R / T64 + E) * p.ntiles, ctx->stream);
  if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "fp32 gate/up: %s", hipGetErrorString(e));
  if (wd == nullptr) return MOE_OK;  // gate/up alone (recompute)
  P32 q{};
  q.a0 = h; q.lda = F;
  q.b0 = wd; q.ldb = d; q.b_gstride = (long long)F * d;
  q.c0 = yp; q.ldc = d;
  q.offsets = offsets; q.E = E; q.N = d; q.K = F; q.kseg = F;
  q.ntiles = (d + T64 - 1) / T64;
  e = run<FWD_DOWN>(q, (R / T64 + E) * q.ntiles, ctx->stream);
  if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "fp32 down: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_internal_ffn_bwd_f32(moe_ctx* ctx, const float* xp, const float* wg,
                                    const float* wu, const float* wd, const int32_t* offsets,
                                    const float* g, const float* u, const float* h,
                                    const float* dyp, int E, int R, int d, int F, float* dg,
                                    float* du, float* dxp, float* dwg, float* dwu, float* dwd) {
  hipError_t e;
  {
    P32 p{};
    p.a0 = dyp; p.lda = d;
    p.b0 = wd; p.ldb = d; p.b_gstride = (long long)F * d;
    p.c0 = dg; p.c1 = du; p.ldc = F;
    p.aux0 = g; p.aux1 = u;
    p.offsets = offsets; p.E = E; p.N = F; p.K = d; p.kseg = d;
    p.ntiles = (F + T64 - 1) / T64;
    e = run<DGRAD_DOWN>(p, R > 0 ? (R / T64 + E) * p.ntiles : 0, ctx->stream);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "fp32 down dgrad: %s", hipGetErrorString(e));
  }
  {
    P32 p{};
    p.a0 = h; p.lda = F;
    p.b0 = dyp; p.ldb = d;
    p.c0 = dwd; p.ldc = d; p.c_gstride = (long long)F * d;
    p.offsets = offsets; p.E = E; p.M = F; p.N = d;
    p.ntiles = (d + T64 - 1) / T64;
    p.mtiles = (F + T64 - 1) / T64;
    e = run<WGRAD_DOWN>(p, E * p.ntiles * p.mtiles, ctx->stream);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "fp32 down wgrad: %s", hipGetErrorString(e));
  }
  {
    P32 p{};
    p.a0 = dg; p.a1 = du; p.lda = F;
    p.b0 = wg; p.b1 = wu; p.ldb = F; p.b_gstride = (long long)d * F;
    p.c0 = dxp; p.ldc = d;
    p.offsets = offsets; p.E = E; p.N = d; p.K = 2 * F; p.kseg = F;
    p.ntiles = (d + T64 - 1) / T64;
    e = run<DGRAD_UP>(p, R > 0 ? (R / T64 + E) * p.ntiles : 0, ctx->stream);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "fp32 gate/up dgrad: %s", hipGetErrorString(e));
  }
  {
    P32 p{};
    p.a0 = xp; p.lda = d;
    p.b0 = dg; p.b1 = du; p.ldb = F;
    p.c0 = dwg; p.c1 = dwu; p.ldc = F; p.c_gstride = (long long)d * F;
    p.offsets = offsets; p.E = E; p.M = d; p.N = F;
    p.ntiles = (F + T64 - 1) / T64;
    p.mtiles = (d + T64 - 1) / T64;
    e = run<WGRAD_UP>(p, E * p.ntiles * p.mtiles, ctx->stream);
    if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "fp32 gate/up wgrad: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}
