// Chunked UA prefill (gfx950) -- kernels follow.
#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

size_t prefill_ws_bytes(const LayerArgs& a, int n_tokens, int max_seg_cap) { return 256; }

hipError_t launch_prefill(const LayerArgs& a, const Control& ctl, int n_tokens, int max_seg_cap, void* scratch,
                          size_t scratch_bytes, hipStream_t st) {
  return hipErrorNotSupported;
}

}  // namespace ua
