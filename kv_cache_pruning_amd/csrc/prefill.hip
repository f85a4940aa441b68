// Chunked UA prefill (gfx950) -- kernels follow.
#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

size_t prefill_ws_bytes(const LayerArgs& a, int n_tokens, int max_seg_cap) { return 256; }

hipError_t launch_prefill(const LayerArgs& a, int n_tokens, void* ws, size_t ws_bytes, hipStream_t st) {
  return hipErrorNotSupported;
}

}  // namespace ua
