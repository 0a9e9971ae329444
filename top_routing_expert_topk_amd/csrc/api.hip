// Status text, version and workspace sizes of libmoe.so.
#include "moe_internal.h"

using namespace moe;

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

extern "C" int moe_version(void) { return 100; }

extern "C" size_t moe_workspace_size(int op, int T, int d, int h, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  switch (op) {
    case MOE_OP_ROUTER: return d < 1 ? 0 : router_ws(T, d, E);
    case MOE_OP_PERMUTE: return permute_ws(T, k, E);
    case MOE_OP_FFN: return (h < 1 || d < 1) ? 0 : ffn_ws(T, d, h, E, k);
    case MOE_OP_FFN_BWD:
      return (h < 1 || d < 1 || E > kMaxE) ? 0 : ffn_bwd_layout(T, d, h, E, k).total;
    case MOE_OP_ROUTER_BWD: return (d < 1 || E > kMaxE) ? 0 : router_bwd_ws(T, d, E);
    default: return 0;
  }
}
