// Launchers of kernel classes this build does not provide yet.  The planner
// never routes work to them (class_available returns false).
#include "../launch.h"

namespace rpa {

hipError_t launch_mla(const DevPlan&, const void*, const void*, Strides, void*, float*,
                      hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace rpa
