// Which specialised kernel classes the compiled library provides.  Pure C++ so the
// planner links without HIP.
#include "plan.h"

namespace rpa {

bool class_available(int32_t kernel_class, const rpa_attn_config& cfg) {
  (void)cfg;
  switch (kernel_class) {
    case KC_GENERIC: return true;
    case KC_DECODE: return true;
    case KC_PREFILL: return true;
    case KC_MLA: return true;
    default: return false;
  }
}

}  // namespace rpa
