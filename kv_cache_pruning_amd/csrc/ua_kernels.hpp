// Internal kernel-argument structs and launcher declarations (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

namespace ua {

// Upper limits the kernels are written for (checked on the host).
constexpr int kMaxHkv = 64;
constexpr int kMaxRank = 64;
constexpr int kMaxSeg = 65536;
constexpr int kMaxDModel = 16384;

struct LayerArgs {
  // shape
  int B, H_q, H_kv, d, D_model, r, terms;
  int bf16;    // q/k/v/x/weights/cache dtype is bf16 (else fp32)
  int y_bf16;  // y dtype is bf16 (else fp32)
  float scale;
  double rope_base;
  double inv_freq[64];  // rope_base^(-2i/d), i < d/2, formed in fp64 on the host
  // weights
  const void* W_dec;
  const float* b_dec;
  const void* W_dn;
  const void* W_up;
  const float* b_up;
  // tokens
  const void* q;
  const void* k;
  const void* v;
  const void* x;
  // cache
  void* K;
  void* V;
  float* lam;
  float* lk;
  const int64_t* seg_off;
  int32_t* seg_len;
  const int32_t* seg_cap;
  int32_t* next_pos;
  int32_t* status;
  int64_t total_slots;
  // output
  void* y;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Control words of a workspace: counters and flags that must be zero before
// the first call; every call returns them to zero, except the call counter at
// glob[kGlobSeq] (prefill tags its carry words with it) and the decode words
// that the decode step's first launch clears itself.  The fixed part sits at
// the front of the workspace, the compaction flags at its end (see
// workspace.hip), so calls on caches of different sizes can share one.
constexpr int kGlobTicket = 0;   // compaction: next work item
constexpr int kGlobArrive = 32;  // compaction: workgroups done (own cache line)
constexpr int kGlobSeq = 64;     // prefill: calls made (tags the carry words)
constexpr int kGlobInts = 128;

struct Control {
  int* dec_cnt;              // [S]           decode: arrivals per segment
  int* cmp_state;            // [max_chunks]  compaction: (count or prefix) << 2 | flag
  int* cmp_loaded;           // [max_chunks]  compaction: the chunk's rows are in registers
  unsigned long long* dec_state;  // [max_chunks]  decode tiles: (count or prefix) << 2 | flag
  int* glob;                 // [kGlobInts]   ticket, arrivals, call counter (one cache line each)
  int cmp_chunk;             // entries per compaction chunk
  int max_chunks;
};

int compact_chunk_entries(const LayerArgs& a);
size_t control_bytes(const LayerArgs& a);       // fixed part at the front
size_t control_tail_bytes(const LayerArgs& a);  // compaction flags at the end
Control control_carve(const LayerArgs& a, void* ws, size_t ws_bytes);

// Decode scratch (after the control block) plus the counters it uses.  The
// token launch writes the per-sequence quantities and the tile records, and
// clears the per-segment counters and look-back words the tile launch uses.
struct DecodeWs {
  int* cnt;        // [S]  arrivals per segment (control block; unused by decode)
  int* segtk;      // [S]  tile tickets per segment
  int* ntiles;     // [1]  tiles of the step
  int4* map;       // [max_tiles, 2]  per tile: {segment, tile of the segment, length, tiles of the segment},
                   //                 {record of the segment's first tile, offset low, offset high, 0}
  float* tq;       // [B, H_q, d]  rotated queries
  float* tkey;     // [B * H_kv, d]  stored new keys (rounded like the cache)
  uint16_t* tqh;   // [B, H_q, d]  bf16 caches: rotated queries, high bf16 part
  uint16_t* tql;   // [B, H_q, d]  and low part (the rest of the fp32 value, rounded)
  uint16_t* tkb;   // [B * H_kv, d]  bf16 caches: the stored new keys as bf16
  float* zdec;     // [B, 4, 3 * H_kv + r]  x [W_dec | W_dn] over four slices of the rows (summed by the readers)
  float* part_o;   // [max_tiles, G, d]   partials of segments held by several tiles
  float* part_ml;  // [max_tiles, G, 2]   max (log2 units), sum
  int max_tiles;
};

size_t decode_ws_bytes(const LayerArgs& a, int tile_entries);
int decode_tile_entries(int d, int g, bool bf16);  // g: query heads per KV head
DecodeWs decode_ws_carve(const LayerArgs& a, const Control& ctl, void* scratch, int tile_entries);
// One decode step; with compact, the in-place compaction of every segment in
// the same launch (kept: optional kept-index output).
hipError_t launch_decode(const LayerArgs& a, const DecodeWs& w, const Control& ctl, float tau, bool compact,
                         int32_t* kept, hipStream_t st);

// Compaction
hipError_t launch_compact(const LayerArgs& a, const Control& ctl, float tau, int32_t* kept, hipStream_t st);

// Prefill (its sync words live in its scratch and are cleared by the call)
size_t prefill_ws_bytes(const LayerArgs& a, int n_tokens, int max_seg_cap);
// Backward of the decay-mask and attention part for one training chunk per
// sequence (token-major arrays, N tokens); the workspace holds Lambda and
// dLambda (N x N fp32 per segment) and two [B, N, H_q] vectors.
size_t backward_ws_bytes(int B, int Hq, int Hkv, int N);
hipError_t launch_backward(int B, int Hq, int Hkv, int D, int N, int terms, float scale, bool bf16, const void* qt,
                           const void* kt, const void* v, const float* lq, const float* lk, const float* lb,
                           const float* dO, float* dq, float* dk, float* dv, float* dlq, float* dlk, float* dlb,
                           void* ws, hipStream_t st);

// In-place RMS normalisation of nq head rows of q and nk of k (d elements each).
hipError_t launch_qk_norm(int d, bool bf16, void* q, const float* wq, int64_t nq, void* k, const float* wk, int64_t nk,
                          float eps, hipStream_t st);

// Prefill of n_tokens per sequence.  Token t of sequence b is row b * ld + t0 + t
// of q, k, v, x and y; log_p (-inf: none) keeps entries whose bias has fallen
// below it out of the softmax.
// cu (device, [B + 1], or null) makes the call variable-length: sequence b
// appends cu[b + 1] - cu[b] <= n_tokens tokens, packed at rows cu[b] .. of the
// total rows of q, k, v, x and y (ld and t0 unused).
hipError_t launch_prefill(const LayerArgs& a, const Control& ctl, int n_tokens, int max_seg_cap, void* scratch,
                          size_t scratch_bytes, hipStream_t st, float log_p, int ld, int t0,
                          const int* cu = nullptr, int total = 0);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// Workgroups of a kernel that fit on the current GPU at once, from the
// runtime's occupancy figure, cached per (kernel, device).
template <typename Kern>
inline hipError_t resident_workgroups(Kern kern, int threads, int* out) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int>, int> cache;
  const void* fn = reinterpret_cast<const void*>(kern);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(fn, threads, dev);
  {
    std::lock_guard<std::mutex> lk(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) {
      *out = it->second;
      return hipSuccess;
    }
  }
  int per_cu = 0, cus = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *out = per_cu > 0 && cus > 0 ? per_cu * cus : 0;
  if (*out > 0) {
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = *out;
  }
  return hipSuccess;
}

}  // namespace ua
