// prefill.hip -- placeholder until the MFMA chunked-prefill kernel lands.
#include "pkv_launch.h"

namespace pkv {

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
