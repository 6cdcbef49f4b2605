// Library-wide host code: error strings, device properties, workspace sizes.
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"

namespace moe {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

moe_status fail(moe_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

moe_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    return fail(MOE_ERR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
  }
  return MOE_OK;
}

int num_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace moe

using namespace moe;

extern "C" const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

extern "C" const char* moe_last_error(void) { return g_last_error.c_str(); }

extern "C" moe_status moe_workspace_size(moe_op op, const moe_mlp_desc* desc, int64_t R, int64_t T,
                                         int E, int k, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "moe_workspace_size: bytes is NULL");
  *bytes = 0;
  switch (op) {
    case MOE_OP_PERMUTE:
      if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E)
        return fail(MOE_ERR_INVALID_ARG, "moe_workspace_size(PERMUTE): bad T/E/k");
      *bytes = permute_workspace_bytes(T, E, k);
      return MOE_OK;
    case MOE_OP_MLP_FWD:
    case MOE_OP_MLP_BWD: {
      if (!desc || R < 0) return fail(MOE_ERR_INVALID_ARG, "moe_workspace_size: desc NULL or R < 0");
      moe_status s = validate_desc(*desc, op == MOE_OP_MLP_BWD);
      if (s != MOE_OK) return s;
      *bytes = op == MOE_OP_MLP_FWD ? mlp_fwd_workspace_bytes(*desc, R) : mlp_bwd_workspace_bytes(*desc, R);
      return MOE_OK;
    }
    case MOE_OP_GROUPED_GEMM:
      *bytes = grouped_gemm_workspace_bytes();
      return MOE_OK;
    case MOE_OP_ROUTER_BWD:
      if (!desc || T < 0 || desc->E < 1 || desc->E > MOE_MAX_EXPERTS || desc->H < 1)
        return fail(MOE_ERR_INVALID_ARG, "moe_workspace_size(ROUTER_BWD): desc NULL or bad T/E/H");
      *bytes = router_bwd_workspace_bytes(T, desc->H, desc->E);
      return MOE_OK;
  }
  return fail(MOE_ERR_INVALID_ARG, "moe_workspace_size: unknown op");
}
