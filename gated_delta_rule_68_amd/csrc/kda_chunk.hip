// Chunked prefill arm (not built yet: the host never selects it).
#include "kda_internal.h"

namespace kda {

const bool kChunkedArmBuilt = false;

size_t chunked_workspace_bytes(int, int, int, int, bool) { return 0; }

hipError_t launch_chunked(const MixerArgs&) { return hipErrorNotSupported; }

}  // namespace kda
