// peak.hip — sustained bf16 matrix-core rate of this GPU, for measurement.
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on register
// operands into four independent accumulators: no memory traffic, no LDS,
// no barriers.  The rate it reaches is the ceiling the grouped GEMMs could
// approach at the clock the chip holds under this load, beside the published
// dense peak.
#include <hip/hip_runtime.h>

#include "common.h"

using namespace moe;

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// a_val, b_val: every operand element (as bf16); each MFMA adds 16·a·b to
// every accumulator element, so sink[thread] = 64 · 16 · a · b · iters
// exactly while that stays below 2^24.
__global__ void __launch_bounds__(256) mfma_peak_kernel(float a_val, float b_val, int iters,
                                                        float* __restrict__ sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)a_val;
    b[i] = (__bf16)b_val;
  }
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

using namespace moe_host;

extern "C" moe_status moe_mfma_peak_probe(moe_ctx* ctx, int blocks, int iters, float a, float b,
                                          float* sink) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, blocks >= 1 && blocks <= (1 << 20) && iters >= 1,
              "moe_mfma_peak_probe: bad blocks=%d iters=%d", blocks, iters);
  MOE_REQUIRE_PTR(ctx, sink);
  mfma_peak_kernel<<<blocks, 256, 0, ctx->stream>>>(a, b, iters, sink);
  return check_launch(ctx, "moe_mfma_peak_probe");
}
