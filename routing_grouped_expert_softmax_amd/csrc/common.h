// common.h — internal helpers shared by the HIP sources of the MoE library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <initializer_list>
#include <cstdio>
#include <string>
#include <utility>
#include <vector>

#include "../../include/moe.h"

// Event pairs recorded around the launches of one kernel id while profiling.
struct moe_prof_slot {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  int used = 0;
};

struct moe_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::string last_error;
  bool prof = false;
  moe_prof_slot slots[MOE_K_COUNT];
};

// Records a start event on construction and a stop event on destruction
// around a launch of kernel `id`, when the context is profiling.
struct moe_prof_scope {
  moe_ctx* c;
  moe_prof_slot* s = nullptr;
  moe_prof_scope(moe_ctx* ctx, int id) : c(ctx) {
    if (!c || !c->prof) return;
    s = &c->slots[id];
    if (s->used == (int)s->ev.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
        s = nullptr;
        return;
      }
      s->ev.emplace_back(a, b);
    }
    // a failed record leaves this launch untimed (the pair is reused)
    if (hipEventRecord(s->ev[s->used].first, c->stream) != hipSuccess) s = nullptr;
  }
  ~moe_prof_scope() {
    if (!s) return;
    if (hipEventRecord(s->ev[s->used].second, c->stream) == hipSuccess) s->used++;
  }
};

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Packs two floats into one dword of two bf16 (lo = a).
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, size_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, size_t i, float v) { p[i] = f2bf(v); }
};

// v_rcp_f32 (about 1 ulp) instead of an IEEE divide: the divide expansion
// needs several temporaries per element, which the epilogues cannot afford
// with a full accumulator tile live.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

}  // namespace moe

// ---------------------------------------------------------------- host side
namespace moe_host {

inline moe_status fail(moe_ctx* ctx, moe_status st, const char* fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    ctx->last_error = buf;
  }
  return st;
}

inline moe_status check_launch(moe_ctx* ctx, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(ctx, MOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t esize(moe_dtype dt) { return dt == MOE_F32 ? 4 : 2; }

// Compute units of the current device (cached per device; 256 if unknown).
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// One output array of a call: its device address range.  NULL or empty
// arrays take part in no overlap.
struct OutSpan {
  const void* p;
  size_t bytes;
  const char* name;
};

// Every pair of a call's outputs must be disjoint (a kernel may write them
// in any order, so overlapping outputs would race).
inline moe_status check_disjoint(moe_ctx* ctx, const char* fn, std::initializer_list<OutSpan> outs) {
  for (const OutSpan* a = outs.begin(); a != outs.end(); ++a) {
    if (a->p == nullptr || a->bytes == 0) continue;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a->p), a1 = a0 + a->bytes;
    for (const OutSpan* b = a + 1; b != outs.end(); ++b) {
      if (b->p == nullptr || b->bytes == 0) continue;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(b->p), b1 = b0 + b->bytes;
      if (a0 < b1 && b0 < a1)
        return fail(ctx, MOE_ERR_INVALID_ARGUMENT, "%s: outputs %s and %s overlap", fn, a->name, b->name);
    }
  }
  return MOE_OK;
}

}  // namespace moe_host

// Rejects the call when two of its outputs overlap.
#define MOE_REQUIRE_DISJOINT(ctx, fn, ...)                                        \
  do {                                                                            \
    const moe_status st_dj_ = moe_host::check_disjoint((ctx), (fn), {__VA_ARGS__}); \
    if (st_dj_ != MOE_OK) return st_dj_;                                          \
  } while (0)

#define MOE_CHECK_CTX(ctx) \
  do {                     \
    if (!(ctx)) return MOE_ERR_INVALID_ARGUMENT; \
  } while (0)

#define MOE_REQUIRE(ctx, cond, ...)                                               \
  do {                                                                            \
    if (!(cond)) return moe_host::fail((ctx), MOE_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

#define MOE_REQUIRE_PTR(ctx, p) \
  MOE_REQUIRE(ctx, (p) != nullptr && moe_host::aligned16(p), "%s: null or not 16-byte aligned", #p)

// A pointer may be null exactly when the array it points to is empty.
#define MOE_REQUIRE_PTR_OR_EMPTY(ctx, p, empty)                                    \
  MOE_REQUIRE(ctx, (empty) || ((p) != nullptr && moe_host::aligned16(p)),         \
              "%s: null or not 16-byte aligned", #p)

#define MOE_REQUIRE_DTYPE(ctx, dt) \
  MOE_REQUIRE(ctx, (dt) == MOE_F32 || (dt) == MOE_BF16, "unsupported dtype %d", (int)(dt))
