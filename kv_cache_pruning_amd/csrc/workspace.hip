// Workspace layout shared by the three entry points:
//
//   [ fixed control | scratch of the call ... | compaction flags ]
//   ^ ws                                       ^ end of ws - tail
//
// The fixed control words (arrival counters, the ticket, the call counter)
// depend only on B and H_kv; the compaction flags (one
// pair per chunk, so their number depends on total_slots) are carved from
// the END of the workspace.  Layers of one shape whose caches differ in size
// can then share one workspace sized for the largest: no call's scratch ever
// overlaps another call's control words.  The control words are zero before
// the first call and every call leaves them zero (the call counter aside; the
// decode step clears its own counters and look-back words in its first
// launch); prefill keeps its own sync words in its scratch and clears them at
// the start of each call.

#include <algorithm>

#include "ua_kernels.hpp"

namespace ua {

int compact_chunk_entries(const LayerArgs& a) {
  const int rb = a.d * (a.bf16 ? 2 : 4);
  return rb <= 128 ? 256 : (rb <= 256 ? 128 : 64);
}

// Flags for compaction chunks and for the tiles of a decode step that compacts
// in the same launch (the finer of the two).
static int64_t compact_max_chunks(const LayerArgs& a) {
  const int unit = std::min(compact_chunk_entries(a), decode_tile_entries(a.d, a.H_q / a.H_kv, a.bf16 != 0));
  return a.total_slots / unit + (int64_t)a.B * a.H_kv + 1;
}

static size_t fixed_layout(const LayerArgs& a, Control* c, char* base) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  size_t n = 0;
  auto take = [&](size_t bytes) {
    int* q = base ? reinterpret_cast<int*>(base + n) : nullptr;
    n += align_up(bytes, 256);
    return q;
  };
  int* dec_cnt = take(sizeof(int) * S);
  int* glob = take(sizeof(int) * kGlobInts);
  if (c) {
    c->dec_cnt = dec_cnt;
    c->glob = glob;
  }
  return n;
}

size_t control_bytes(const LayerArgs& a) { return fixed_layout(a, nullptr, nullptr); }

size_t control_tail_bytes(const LayerArgs& a) {
  const int64_t mc = compact_max_chunks(a);
  return 2 * align_up(sizeof(int) * mc, 256) + align_up(sizeof(unsigned long long) * mc, 256);
}

Control control_carve(const LayerArgs& a, void* ws, size_t ws_bytes) {
  Control c{};
  char* base = reinterpret_cast<char*>(ws);
  fixed_layout(a, &c, base);
  const int64_t mc = compact_max_chunks(a);
  const size_t one = align_up(sizeof(int) * mc, 256);
  char* tail = base + (ws_bytes / 256 * 256) - control_tail_bytes(a);  // callers check ws_bytes covers every part
  c.cmp_state = reinterpret_cast<int*>(tail);
  c.cmp_loaded = reinterpret_cast<int*>(tail + one);
  c.dec_state = reinterpret_cast<unsigned long long*>(tail + 2 * one);
  c.cmp_chunk = compact_chunk_entries(a);
  c.max_chunks = (int)mc;
  return c;
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = i; k < n16; k += stride) p[k] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  const size_t want = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<uint4*>(p), n16,
                     reinterpret_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace ua
