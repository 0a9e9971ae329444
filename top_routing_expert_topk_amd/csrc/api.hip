// Status text, version and workspace sizes of libmoe.so, and the copy to
// the host behind the debug build's permutation checks.
#include <vector>

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

extern "C" size_t moe_expert_output_bytes(int dtype, int rows, int d) {
  if (rows < 0 || d < 1) return 0;
  if (dtype == MOE_F32) return (size_t)rows * d * sizeof(float);
  if (dtype != MOE_BF16 || (d % kYBlock) != 0) return 0;
  static_assert(MOE_YQ_ROW_BYTES(64) == 2 * 64 + 16, "row bytes");
  return (size_t)rows * yq_row_bytes(d);
}

extern "C" size_t moe_workspace_size(int op, int T, int d, int h, int E, int k) {
  // no call of this build takes more than kMaxE experts (the router's token
  // tile would round down to zero rows past it)
  if (T < 0 || E < 1 || k < 1 || E > kMaxE) return 0;
  switch (op) {
    case MOE_OP_ROUTER: return d < 1 ? 0 : router_ws(T, d, E);
    case MOE_OP_PERMUTE: return permute_ws(T, k, E);
    case MOE_OP_FFN: return (h < 1 || d < 1) ? 0 : ffn_ws(T, d, h, E, k);
    case MOE_OP_FFN_BWD: return (h < 1 || d < 1) ? 0 : ffn_bwd_layout(T, d, h, E, k).total;
    case MOE_OP_ROUTER_BWD: return d < 1 ? 0 : router_bwd_ws(T, d, E);
    default: return 0;
  }
}

namespace moe {

int debug_check(hipStream_t s, const int32_t* offsets, int E, const int32_t* sorted_token,
                const int32_t* dest_row, int T, int k) {
  const long slots = (long)T * k;
  if (slots <= 0) return MOE_OK;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_LAUNCH;
  std::vector<int32_t> off, st, dr;
  long R = slots;
  if (offsets) {
    off.resize((size_t)E + 1);
    if (hipMemcpy(off.data(), offsets, off.size() * sizeof(int32_t), hipMemcpyDeviceToHost) !=
        hipSuccess)
      return MOE_ERR_LAUNCH;
    R = off[E];
    if (R < 0 || R > slots) return MOE_ERR_INVALID;
  }
  if (sorted_token && R > 0) {
    st.resize((size_t)R);
    if (hipMemcpy(st.data(), sorted_token, st.size() * sizeof(int32_t),
                  hipMemcpyDeviceToHost) != hipSuccess)
      return MOE_ERR_LAUNCH;
  }
  if (dest_row) {
    dr.resize((size_t)slots);
    if (hipMemcpy(dr.data(), dest_row, dr.size() * sizeof(int32_t), hipMemcpyDeviceToHost) !=
        hipSuccess)
      return MOE_ERR_LAUNCH;
  }
  const int32_t* stp = sorted_token ? (R > 0 ? st.data() : off.data()) : nullptr;
  return moe_check_permutation(offsets ? off.data() : nullptr, E, stp,
                               dest_row ? dr.data() : nullptr, T, k);
}

}  // namespace moe
