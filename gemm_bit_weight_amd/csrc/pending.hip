// The E4M3-B16 grouped GEMM (bf16 MFMA) is not built yet.
#include "common.hpp"

namespace gbw {
struct MoeArgs;
int launch_moe_bf16(const MoeArgs&, const gbw_act*, const gbw_weight*, int, hipStream_t) {
  return fail(GBW_E_UNSUPPORTED, "moe_grouped_gemm: E4M3-B16 path not built");
}
}  // namespace gbw
