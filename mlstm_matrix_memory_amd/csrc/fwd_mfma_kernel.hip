// Chunkwise forward on bf16 MFMA -- not yet enabled.
#include "mlstm_internal.h"

namespace mlstm {
bool mfma_fwd_supported(const FwdArgs&) { return false; }
size_t mfma_fwd_workspace_bytes(const FwdArgs&) { return 0; }
hipError_t launch_fwd_mfma(const FwdArgs&) { return hipErrorNotSupported; }
}  // namespace mlstm
