#include "lrt_common.hpp"
#include "lrt_internal.hpp"
namespace lrt {
int fwd_kda(const FwdArgs&) { return -2; }
}  // namespace lrt
