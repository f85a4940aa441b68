// Workspace control block: counters and flags of the decode and compaction
// kernels.  They are zero before the first call and every call leaves them
// zero, so one workspace can serve decode, prefill and compaction calls
// issued in order on one stream (prefill keeps its own sync words in its
// scratch and clears them at the start of each call).

#include "ua_kernels.hpp"

namespace ua {

int compact_chunk_entries(const LayerArgs& a) {
  const int rb = a.d * (a.bf16 ? 2 : 4);
  return rb <= 128 ? 256 : (rb <= 256 ? 128 : 64);
}

static size_t control_layout(const LayerArgs& a, Control* c, char* base) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int ch = compact_chunk_entries(a);
  const int64_t mc = a.total_slots / ch + S + 1;
  size_t n = 0;
  auto take = [&](size_t bytes) {
    int* q = base ? reinterpret_cast<int*>(base + n) : nullptr;
    n += align_up(bytes, 256);
    return q;
  };
  int* dec_cnt = take(sizeof(int) * S);
  int* dec_cntb = take(sizeof(int) * a.B);
  int* cmp_state = take(sizeof(int) * mc);
  int* cmp_loaded = take(sizeof(int) * mc);
  int* cmp_done = take(sizeof(int) * S);
  int* cmp_glob = take(sizeof(int) * 2);
  if (c) {
    c->dec_cnt = dec_cnt;
    c->dec_cntb = dec_cntb;
    c->cmp_state = cmp_state;
    c->cmp_loaded = cmp_loaded;
    c->cmp_done = cmp_done;
    c->cmp_glob = cmp_glob;
    c->cmp_chunk = ch;
    c->max_chunks = (int)mc;
  }
  return n;
}

size_t control_bytes(const LayerArgs& a) { return control_layout(a, nullptr, nullptr); }

Control control_carve(const LayerArgs& a, void* ws) {
  Control c{};
  control_layout(a, &c, reinterpret_cast<char*>(ws));
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
