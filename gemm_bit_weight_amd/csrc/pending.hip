// Entry points whose kernels are not built yet: they validate nothing and
// report GBW_E_UNSUPPORTED.
#include "common.hpp"

namespace gbw {
size_t ws_moe_route(int64_t, int64_t) { return 0; }
size_t ws_moe_gemm(int64_t, int64_t, int32_t) { return 0; }
}  // namespace gbw

using namespace gbw;

extern "C" int moe_route(const float*, int64_t, int32_t, int32_t, int32_t*, float*, int32_t*, int32_t*, int32_t*,
                         void*, size_t, void*) {
  return fail(GBW_E_UNSUPPORTED, "moe_route: not built");
}
extern "C" int moe_grouped_gemm(int32_t, int64_t, int32_t, const int32_t*, const int32_t*, const int32_t*,
                                const float*, const gbw_act*, const gbw_weight*, const gbw_moe_out*, int32_t,
                                void*, size_t, void*) {
  return fail(GBW_E_UNSUPPORTED, "moe_grouped_gemm: not built");
}
