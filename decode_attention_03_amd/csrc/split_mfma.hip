// split_mfma.hip -- grouped-query split stage on the gfx950 matrix cores.
#include "dev_common.h"

namespace fd {

bool split_mfma_supported(int, int, int) { return false; }

hipError_t launch_split_mfma(const SplitArgs &, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fd
