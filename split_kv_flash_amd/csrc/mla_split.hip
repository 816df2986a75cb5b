// Shared-latent (multi-head latent attention, absorbed form) split kernel.
#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

bool latent_supported(const sk_desc_t&) { return false; }

sk_status_t latent_split_launch(const SplitLaunch&, bool, const void**, int*, int*) {
  return SK_ERR_UNSUPPORTED;
}

}  // namespace sk
