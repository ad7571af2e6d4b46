// context.hip — context, stream, workspace and status entry points of the C ABI.
#include "common.h"

extern "C" {

moe_status moe_create(int device, void* hip_stream, moe_ctx** out) {
  if (!out) return MOE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n)
    return MOE_ERR_INVALID_ARGUMENT;
  moe_ctx* c = new (std::nothrow) moe_ctx();
  if (!c) return MOE_ERR_HIP;
  c->device = device;
  c->stream = reinterpret_cast<hipStream_t>(hip_stream);
  *out = c;
  return MOE_OK;
}

moe_status moe_destroy(moe_ctx* ctx) {
  MOE_CHECK_CTX(ctx);
  for (auto& s : ctx->slots)
    for (auto& e : s.ev) {
      hipEventDestroy(e.first);
      hipEventDestroy(e.second);
    }
  delete ctx;
  return MOE_OK;
}

moe_status moe_profile_enable(moe_ctx* ctx, int on) {
  MOE_CHECK_CTX(ctx);
  ctx->prof = on != 0;
  if (ctx->prof)
    for (auto& s : ctx->slots) s.used = 0;
  return MOE_OK;
}

moe_status moe_profile_query(moe_ctx* ctx, int id, int* launches, double* total_ms) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, id >= 0 && id < MOE_K_COUNT && launches && total_ms, "bad profile query");
  const moe_prof_slot& s = ctx->slots[id];
  double sum = 0;
  for (int i = 0; i < s.used; ++i) {
    if (hipEventSynchronize(s.ev[i].second) != hipSuccess)
      return moe_host::fail(ctx, MOE_ERR_HIP, "profile: event wait failed");
    float ms = 0;
    if (hipEventElapsedTime(&ms, s.ev[i].first, s.ev[i].second) != hipSuccess)
      return moe_host::fail(ctx, MOE_ERR_HIP, "profile: elapsed time failed");
    sum += ms;
  }
  *launches = s.used;
  *total_ms = sum;
  return MOE_OK;
}

const char* moe_kernel_name(int id) {
  static const char* names[MOE_K_COUNT] = {
      "router_logits", "topk_hist", "expert_scan", "rank", "permute", "gemm_up_swiglu",
      "gemm_down", "combine", "combine_bwd", "route_bwd", "gemm_dgrad_down_swiglu",
      "gemm_wgrad_down", "gemm_dgrad_up", "gemm_wgrad_up", "permute_bwd", "router_wgrad",
      "mx_quantize", "route_stats", "aux_loss_bwd", "grad_norms", "router_dense_bwd"};
  if (id < 0 || id >= MOE_K_COUNT) return "unknown";
  return names[id];
}

moe_status moe_set_stream(moe_ctx* ctx, void* hip_stream) {
  MOE_CHECK_CTX(ctx);
  ctx->stream = reinterpret_cast<hipStream_t>(hip_stream);
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(const moe_ctx* ctx) {
  if (!ctx) return "null context";
  return ctx->last_error.c_str();
}

moe_status moe_set_workspace(moe_ctx* ctx, void* ws, size_t bytes) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) == 0,
              "workspace must be 256-byte aligned");
  ctx->ws = ws;
  ctx->ws_bytes = ws ? bytes : 0;
  return MOE_OK;
}

}  // extern "C"
