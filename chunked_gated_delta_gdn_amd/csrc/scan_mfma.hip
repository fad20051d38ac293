// Matrix-core (MFMA) scan for bf16 inputs at K = V = 128, C = 64.
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {

bool mfma_scan_available(int, int, int, int) { return false; }

hipError_t launch_scan_mfma(int, int, int, int, bool, const ScanArgs &, hipStream_t,
                            bool *handled) {
    *handled = false;
    return hipSuccess;
}

}  // namespace gdn
