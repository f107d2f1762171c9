// WKV7 chunked-parallel prefill (ALGO_CHUNKED) -- not built yet.
#include "wkv7_internal.h"

namespace wkv7 {

const bool kChunkedAvailable = false;

size_t chunked_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_chunked(const ForwardArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace wkv7
