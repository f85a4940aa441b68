// Internal kernel-argument structs and launcher declarations (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

// Decode workspace regions (device pointers into the caller's workspace).
struct DecodeWs {
  float* qt;      // [B, H_q, d]   rotated queries
  float* kt;      // [S, d]        stored new keys (cache-rounded), fp32
  float* gates;   // [S, 4]        lq, lk, lb, unused
  float* gamma;   // [B, H_q, d]   output gate
  int* len_old;   // [S]           segment length before the append
  int* cnt;       // [S]           finished tiles per segment
  float* part_o;  // [max_tiles, G, d]
  float* part_ml; // [max_tiles, G, 2]  running max (log2 units), sum
  int max_tiles;
};

size_t decode_ws_bytes(const LayerArgs& a, int tile_entries);
int decode_tile_entries(int d);
DecodeWs decode_ws_carve(const LayerArgs& a, void* ws, int tile_entries);
hipError_t launch_decode(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st);

// Compaction
size_t compact_ws_bytes(const LayerArgs& a);
hipError_t launch_compact(const LayerArgs& a, float tau, int32_t* kept, void* ws, hipStream_t st);

// Prefill
size_t prefill_ws_bytes(const LayerArgs& a, int n_tokens, int max_seg_cap);
hipError_t launch_prefill(const LayerArgs& a, int n_tokens, void* ws, size_t ws_bytes, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace ua
