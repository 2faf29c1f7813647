// Chunked KDA prefill on bf16 MFMA (d = 128, chunk 64, bf16 io).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

bool prefill_mfma_supported(int, int, int) { return false; }
size_t prefill_mfma_workspace(int, int, int, int, int) { return 0; }
hipError_t launch_prefill_mfma(const LayerArgs&, void*, size_t, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
