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
  delete ctx;
  return MOE_OK;
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
