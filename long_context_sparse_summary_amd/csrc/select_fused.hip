// Instantiations of the fused select (scoring with the cut in each segment's
// last workgroup) for 4 and 8 key slots per lane (segments of up to 4096
// pages), in a translation unit of their own so that the build compiles them
// beside the other selection kernels.
#include "select_impl.h"

namespace moira {
#define MOIRA_FUSED_INST(E)                                                                        \
  template hipError_t launch_fused_select_e<E>(const Dims&, const void*, const void*,             \
                                               const int32_t*, const int32_t*, float,             \
                                               const SelectWs&, const AppendArgs&, bool,          \
                                               const CutArgs&, int32_t*, hipStream_t);
MOIRA_FUSED_INST(4)
MOIRA_FUSED_INST(8)
#undef MOIRA_FUSED_INST
}  // namespace moira
