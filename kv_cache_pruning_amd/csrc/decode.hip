// UA decode step on a ragged, per-KV-head pruned cache (gfx950), two launches,
// optionally with the in-place compaction of every segment in the second.
//
// A decode step ("A Self-Pruning Transformer ...", paperlayer.ai summary,
// section 4.2; ai4snews page, Figure 1 caption): the new token's queries and
// L2-normalised key are rotated (RoPE, angles in fp64); its gates come from x
// W_dec + b_dec; every cached entry that is still live gets the pair term
// (geometric mean of the enabled decays in log space, paperlayer.ai sections
// 4 and 4.1) added to its log-bias; entries that fall below log p are left
// out of the step's softmax and are evicted; the output is the low-rank
// sigmoid gate times the attention output; the new entry is appended.
//
// Launch 1, decode_token_kernel (one workgroup for the tile records, then 4
// per sequence): workgroup 0 numbers the tiles of the step from the segment
// lengths (a tile is TWG consecutive entries of one segment), writes one
// record per tile, clears the per-segment counters and the look-back words of
// the second launch, and reports a length above its capacity (status bit 2;
// then no tile runs).  Workgroup (b, p) forms what depends on the token alone:
// the projections x W_dec and u = x W_dn over a quarter of the rows (readers
// add the quarters), a quarter of the rotated queries (fp32, and for bf16
// caches also as high and low bf16 parts) and of the stored keys (normalised,
// rotated, rounded like the cache); a fifth wave forms the RoPE table of the
// position (fp64 angles) while the projections load.
//
// Launch 2, one four-wave workgroup per tile (decode_tile_mf_kernel for bf16
// caches, decode_tile_kernel for fp32): the tile's key rows, biases and key
// gates are loaded once; every entry gets its q.k products (one per query head
// of the group) and its key similarity in the same pass, the pair term
// updates its log-bias, entries below log p drop out, and an online-softmax
// partial (max, sum, weighted V) is formed per wave and merged across the
// waves in LDS.  With bf16 caches the products run on the matrix cores and V
// is staged in LDS by direct loads; with fp32 caches they run on the vector
// ALUs with the rows in registers.  Every wait below is on a lower tile of
// the same segment.
//  * A one-tile segment combines at once; otherwise each tile publishes its
//    partial before its flag word, and the segment's last tile to arrive
//    merges them.  The combine adds the token's own term and multiplies by the
//    output gate sigmoid(u W_up + b_up).
//  * With COMPACT the survivors move down in place: a tile publishes its live
//    count once every row of the tile is in registers or LDS and looks back
//    over the earlier tiles of its segment for its destination (decoupled
//    look-back); the look-back cannot finish before every earlier tile has
//    published, which orders the stores after the loads they overwrite.  Rows
//    already in place are not rewritten; every survivor's new log-bias is
//    stored.  The segment's last tile appends the new entry after the
//    survivors and writes the length.
//  * Without COMPACT the log-biases are updated in place and the merging tile
//    appends the new entry at the old length.
// No launch reads a length another workgroup of the same launch writes: the
// tile records carry the lengths at the start of the step.
//
// Cross-workgroup data go through relaxed agent-scope atomics (coherent across
// the XCDs without cache-wide write-back or invalidation).

#include <algorithm>

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_coh(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sti_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64_coh(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld64_coh(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kTokThreads = 320;  // two projections of 128 threads each, and one wave for the RoPE table
constexpr int kTokParts = 4;  // token-launch workgroups per sequence
constexpr int kTileThreads = 256;
constexpr int kTileWaves = kTileThreads / 64;
constexpr int kSpinLimitDec = 1 << 22;

// Element t of a bf16 / fp32 row held as raw 16-byte chunks.
template <bool BF16>
__device__ __forceinline__ float chunk_elem(const u32x4& c, int t) {
  if constexpr (BF16) {
    const uint32_t wd = c[t >> 1];
    return (t & 1) ? bf16_hi(wd) : bf16_lo(wd);
  } else {
    return __uint_as_float(c[t]);
  }
}

template <bool BF16>
struct Row8 {
  u32x4 w[BF16 ? 1 : 2];
};

// Loads and stores at a 32-bit byte offset from a uniform base (the
// scalar-base + vector-offset addressing form, no 64-bit address math).
template <typename T>
__device__ __forceinline__ T ld_at(const char* base, uint32_t boff) {
  return *reinterpret_cast<const T*>(base + boff);
}
template <bool BF16>
__device__ __forceinline__ float elem_at(const char* base, uint32_t boff) {
  if constexpr (BF16) {
    return bf16_to_f32(ld_at<uint16_t>(base, boff));
  } else {
    return ld_at<float>(base, boff);
  }
}
template <bool BF16>
__device__ __forceinline__ void row_load_at(Row8<BF16>& r, const char* base, uint32_t boff) {
  r.w[0] = ld_at<u32x4>(base, boff);
  if constexpr (!BF16) r.w[1] = ld_at<u32x4>(base, boff + 16);
}
template <bool BF16>
__device__ __forceinline__ void row_store_at(const Row8<BF16>& r, char* base, uint32_t boff) {
  *reinterpret_cast<u32x4*>(base + boff) = r.w[0];
  if constexpr (!BF16) *reinterpret_cast<u32x4*>(base + boff + 16) = r.w[1];
}

template <bool BF16>
__device__ __forceinline__ void row_zero_if(Row8<BF16>& r, bool zero) {
#pragma unroll
  for (int t = 0; t < (BF16 ? 1 : 2); ++t) r.w[t] = zero ? u32x4{0u, 0u, 0u, 0u} : r.w[t];
}

template <bool BF16>
__device__ __forceinline__ void row_f32(const Row8<BF16>& r, float (&o)[8]) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (i & 1) ? bf16_hi(r.w[0][i >> 1]) : bf16_lo(r.w[0][i >> 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = __uint_as_float(r.w[i >> 2][i & 3]);
  }
}

// Entries per lane group (rows held in registers at once), by head dim and
// query heads per KV head: four keeps a tile's loads in flight together; at
// group size 8 the queries and the weighted-V sums of eight heads leave room
// for two.
constexpr int decode_nb(int d, int g) { return g >= 8 ? 4 : 8; }

template <int D, int NB_>
struct TileShape {
  static constexpr int LPE = D / 8;     // lanes per entry (8 elements each)
  static constexpr int NGW = 64 / LPE;  // entry groups per wave
  static constexpr int NB = NB_;        // entries per group
  static constexpr int TW = NGW * NB;   // entries per wave
  static constexpr int TWG = TW * kTileWaves;
  static_assert(NB <= LPE, "lane c < NB of a group holds entry c's flags");
};

__device__ __forceinline__ int tiles_of(int n, int twg) { return n <= 0 ? 1 : ceil_div(n, twg); }

// All kernel arguments in one struct, read through the kernel-argument
// segment pointer where they are used (separate by-value parameters are all
// loaded at entry and mostly spill).
struct DecodeKArgs {
  LayerArgs a;
  DecodeWs w;
  Control ctl;
  float tau;
  int32_t* kept;
  int twg;
  int resident;  // tile workgroups that fit on the GPU at once (0: unknown)
};

// ---------------------------------------------------------------------------
// launch 1: the token's own quantities, once per sequence; the tile records
// ---------------------------------------------------------------------------
// Partial sums of z[c] = x . M[:, c] for the ncols columns of a row-major [D,
// ncols] matrix by NTH threads (thread t of them): threads take 16-byte column
// chunks (or single columns) and split the rows, every load of a pass in
// flight together; the partials go to s_red (rows [0, NTH)).  gemv_finish
// adds them up after a barrier.
struct GemvPlan {
  int ncols, CWv, nch, npow, R, reff;
  bool vec;
};

template <bool BF16, int NTH>
__device__ __forceinline__ GemvPlan gemv_plan(int ncols) {
  constexpr int CW = BF16 ? 8 : 4;  // elements per 16-byte chunk
  GemvPlan p;
  p.ncols = ncols;
  p.vec = ncols % CW == 0;
  p.CWv = p.vec ? CW : 1;
  p.nch = p.vec ? ncols / CW : ncols;
  p.npow = 1;
  while (p.npow < p.nch) p.npow <<= 1;
  p.R = NTH / p.npow;  // row subsets (>= 1: at most 256 columns)
  p.reff = p.npow <= 64 ? NTH / 64 : p.R;
  return p;
}

struct RopeTable {  // the RoPE table of a position, formed while a gemv's loads fly
  const double* inv_freq;
  int pos, half;
  float *cs, *sn;
};

__device__ __forceinline__ void rope_entry(const RopeTable& rt, int i) {  // fp64 angle
  double sn, cs;
  sincos((double)rt.pos * rt.inv_freq[i], &sn, &cs);
  rt.cs[i] = (float)cs;
  rt.sn[i] = (float)sn;
}

template <bool BF16, int NTH>
__device__ __forceinline__ void gemv_partial(const GemvPlan& p, int t, int r0, int r1, const void* Mv,
                                             const char* xrow, float (*s_red)[8], const RopeTable* rt = nullptr) {
  constexpr int KR = 16;  // rows per thread per pass
  const int lane = t & 63;
  const int wv = t >> 6;
  const char* const mbase = reinterpret_cast<const char*>(Mv);
  const int kc = t & (p.npow - 1), rsub = t / p.npow;
  const bool own = kc < p.nch;
  const int mc0 = own ? kc * p.CWv : 0;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  bool tdone = false;
  for (int rb = r0 + rsub; rb < r1; rb += KR * p.R) {
    float xr[KR];
    u32x4 raw[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const int row = min(rb + q * p.R, r1 - 1);
      xr[q] = elem_at<BF16>(xrow, (uint32_t)row * (BF16 ? 2 : 4));
      const uint32_t e = (uint32_t)(row * p.ncols + mc0) * (BF16 ? 2 : 4);
      if (p.vec) {
        raw[q] = ld_at<u32x4>(mbase, e);
      } else {
        raw[q] = u32x4{__float_as_uint(elem_at<BF16>(mbase, e)), 0u, 0u, 0u};
      }
    }
    if (rt && !tdone && t < rt->half) rope_entry(*rt, t);
    tdone = true;
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const float xv = (own && rb + q * p.R < r1) ? xr[q] : 0.0f;
      if (p.vec) {
#pragma unroll
        for (int e = 0; e < (BF16 ? 8 : 4); ++e) acc[e] = fmaf(xv, chunk_elem<BF16>(raw[q], e), acc[e]);
      } else {
        acc[0] = fmaf(xv, __uint_as_float(raw[q][0]), acc[0]);
      }
    }
  }
  if (rt && !tdone && t < rt->half) rope_entry(*rt, t);  // no rows for this thread
  if (p.npow <= 64) {  // a wave holds every column group: reduce its row subsets in registers
    for (int o = p.npow; o < 64; o <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    if (lane < p.npow) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wv * p.npow + lane][e] = acc[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_red[t][e] = acc[e];
  }
}

__device__ __forceinline__ float gemv_finish(const GemvPlan& p, int c, const float (*s_red)[8]) {
  const int grp = c / p.CWv;
  const int e = c - grp * p.CWv;
  float z = 0.0f;
  for (int rr = 0; rr < p.reff; ++rr) z += s_red[rr * p.npow + grp][e];
  return z;
}

// A rotated query element: fp32, and for bf16 caches also split into a high
// and a low bf16 part (x = hi + lo up to 2^-17 relative) for the matrix cores.
template <bool BF16>
__device__ __forceinline__ void store_query(const DecodeWs& w, int64_t i, float x) {
  w.tq[i] = x;
  if constexpr (BF16) {
    const uint16_t hi = f32_to_bf16(x);
    w.tqh[i] = hi;
    w.tql[i] = f32_to_bf16(x - bf16_to_f32(hi));
  }
}

// Tile numbering order: segments of at least kLongSegTiles tiles first, then
// those of at least two, then the one-tile segments.
constexpr int kLongSegTiles = 8;
constexpr int kMapSegs = 2048;   // segments whose records go through LDS at most
constexpr int kMapTiles = 4096;  // tiles whose segment is looked up in LDS at most

// Dynamic LDS of the token launch: only the map workgroup uses it, and every
// workgroup of the launch allocates it, so it is sized by this layer's
// segments and tile bound rather than by the largest tables.
static size_t token_map_lds(int S, int64_t max_tiles) {
  const size_t segs = (size_t)std::min(S, kMapSegs);
  const size_t tiles = (size_t)std::min<int64_t>(max_tiles, kMapTiles);
  return segs * (sizeof(int64_t) + 2 * sizeof(int)) + tiles * sizeof(int);
}

template <int D, bool BF16>
__global__ __launch_bounds__(kTokThreads) void decode_token_kernel(DecodeKArgs karg) {
  const DecodeKArgs& K = *(const DecodeKArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  constexpr int NT = kTokThreads;
  constexpr int NH = 128;  // threads per projection
  constexpr int HALF = D / 2;
  constexpr int P = kTokParts;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int Hkv = a.H_kv, Hq = a.H_q;
  const int S = a.B * Hkv;

  __shared__ float s_red[NT][8];
  __shared__ float s_cs[HALF], s_sn[HALF];
  __shared__ int s_scan[NT / 64 + 1];
  // the map workgroup's tables, in LDS sized by the launch (token_map_lds):
  // the segments' offsets, first tiles and lengths, and tile -> segment
  extern __shared__ __attribute__((aligned(16))) int64_t s_map[];
  const int mapSegs = min(S, kMapSegs), mapTiles = min(w.max_tiles, kMapTiles);
  int64_t* const s_off = s_map;
  int* const s_first = reinterpret_cast<int*>(s_off + mapSegs);
  int* const s_len = s_first + mapSegs;
  int* const s_seg = s_len + mapSegs;

  if (blockIdx.x == 0) {
    // ---- the tile records of this step, from the lengths at its start: a
    // thread holds S / NT segments (all loaded in one round when there are at
    // most MP), scans their tile counts with the others, then writes its own
    // segments' records
    constexpr int MP = 8;
    const int twg = K.twg;
    const int per = (S + NT - 1) / NT;
    const int sb = min(S, tid * per), se = min(S, sb + per);
    int lenr[MP], capr[MP];
    int64_t offr[MP];
    int mine = 0, mineL = 0, mineM = 0, badl = 0;
    if (per <= MP) {
#pragma unroll
      for (int k = 0; k < MP; ++k) {
        const bool in = sb + k < se;
        lenr[k] = in ? a.seg_len[sb + k] : 0;
        capr[k] = in ? a.seg_cap[sb + k] : 0;
        offr[k] = in ? a.seg_off[sb + k] : 0;
      }
#pragma unroll
      for (int k = 0; k < MP; ++k) {
        if (sb + k < se) {
          const int nt = tiles_of(lenr[k], twg);
          mine += nt;
          mineL += nt >= kLongSegTiles ? nt : 0;
          mineM += (nt >= 2 && nt < kLongSegTiles) ? nt : 0;
          badl |= (lenr[k] < 0 || lenr[k] > capr[k]) ? 1 : 0;
        }
      }
    } else {
      for (int s = sb; s < se; ++s) {
        const int len = a.seg_len[s];
        const int nt = tiles_of(len, twg);
        mine += nt;
        mineL += nt >= kLongSegTiles ? nt : 0;
        mineM += (nt >= 2 && nt < kLongSegTiles) ? nt : 0;
        badl |= (len < 0 || len > a.seg_cap[s]) ? 1 : 0;
      }
    }
    // Longer segments are numbered first: their tiles start in the first
    // round, and the merge that ends each of them overlaps the shorter
    // segments' tiles instead of ending the launch.  A segment's tiles stay
    // consecutive, in segment order within each class.
    int total, totalL, totalM;
    const int run0 = block_exclusive_scan<NT>(mine, s_scan, &total);
    int runL = block_exclusive_scan<NT>(mineL, s_scan, &totalL);
    const int runM0 = block_exclusive_scan<NT>(mineM, s_scan, &totalM);
    int runM = totalL + runM0;
    int runS = totalL + totalM + (run0 - runL - runM0);  // one-tile segments of the threads before
    auto first_of = [&](int nt) {
      int f;
      if (nt >= kLongSegTiles) {
        f = runL;
        runL += nt;
      } else if (nt >= 2) {
        f = runM;
        runM += nt;
      } else {
        f = runS;
        runS += nt;
      }
      return f;
    };
    // A segment whose tiles all fall among the first K.resident records runs
    // without tickets: those workgroups fit on the GPU together, and one that
    // waits on a workgroup not yet started holds no slot that workgroup needs
    // (the later, ticketed workgroups always finish).  Other segments of
    // several tiles take per-segment tickets.
    auto ticketed = [&](int f, int nt) { return (nt > 1 && (K.resident <= 0 || f + nt > K.resident)) ? 1 : 0; };
    const bool bad = __syncthreads_or(badl) != 0;
    if (S <= mapSegs && total <= mapTiles) {
      // the tile -> segment table and the segments' first tile, length and
      // offset into LDS, then the records written evenly by every thread
#pragma unroll
      for (int k = 0; k < MP; ++k) {
        if (sb + k < se) {
          const int nt = tiles_of(lenr[k], twg);
          const int f = first_of(nt);
          s_first[sb + k] = f;
          s_len[sb + k] = lenr[k];
          s_off[sb + k] = offr[k];
          for (int t = 0; t < nt; ++t) s_seg[f + t] = sb + k;
        }
      }
      __syncthreads();
      for (int t = tid; t < total && t < w.max_tiles; t += NT) {  // lengths beyond capacity break the bound
        const int sg = s_seg[t];
        const int f = s_first[sg];
        const int len = s_len[sg];
        const int64_t off = s_off[sg];
        const int nt = tiles_of(len, twg);
        w.map[2 * t + 0] = make_int4(sg, t - f, len, nt);
        w.map[2 * t + 1] = make_int4(f, (int)(uint32_t)(off & 0xffffffff), (int)(off >> 32), ticketed(f, nt));
      }
    } else if (per <= MP) {
#pragma unroll
      for (int k = 0; k < MP; ++k) {
        if (sb + k < se) {
          const int nt = tiles_of(lenr[k], twg);
          const int f = first_of(nt);
          for (int t = 0; t < nt && f + t < w.max_tiles; ++t) {
            w.map[2 * (f + t) + 0] = make_int4(sb + k, t, lenr[k], nt);
            w.map[2 * (f + t) + 1] =
                make_int4(f, (int)(uint32_t)(offr[k] & 0xffffffff), (int)(offr[k] >> 32), ticketed(f, nt));
          }
        }
      }
    } else {
      for (int s = sb; s < se; ++s) {
        const int len = a.seg_len[s];
        const int nt = tiles_of(len, twg);
        const int64_t off = a.seg_off[s];
        const int f = first_of(nt);
        for (int t = 0; t < nt && f + t < w.max_tiles; ++t) {
          w.map[2 * (f + t) + 0] = make_int4(s, t, len, nt);
          w.map[2 * (f + t) + 1] = make_int4(f, (int)(uint32_t)(off & 0xffffffff), (int)(off >> 32), ticketed(f, nt));
        }
      }
    }
    for (int s = sb; s < se; ++s) {
      w.cnt[s] = 0;
      w.segtk[s] = 0;
    }
    if (bad || total > w.max_tiles) {  // a segment length above its capacity: no tile runs
      if (tid == 0) atomicOr(a.status, 4);
      total = 0;
    }
    for (int t = tid; t < total; t += NT) K.ctl.dec_state[t] = 0ull;
    if (tid == 0) *w.ntiles = total;
    return;
  }
  // Workgroup (b, p): part p of P of sequence b's token work.  Every load of
  // the part is issued first: its slice of x and of the rows of W_dec and
  // W_dn, its queries and keys.
  const int b = (blockIdx.x - 1) / P;
  const int p = (blockIdx.x - 1) - b * P;
  const char* const xrow = reinterpret_cast<const char*>(a.x) + (int64_t)b * a.D_model * (BF16 ? 2 : 4);
  const int Dm = a.D_model;
  const int r0 = (p * Dm) / P, r1 = ((p + 1) * Dm) / P;
  const GemvPlan pd = gemv_plan<BF16, NH>(3 * Hkv);
  const GemvPlan pn = gemv_plan<BF16, NH>(a.r);
  // queries: item e = (head, pair) of the sequence, every P-th block of NT items
  constexpr int QI = 4;  // items per thread in flight together
  float q0v[QI], q1v[QI];
#pragma unroll
  for (int j = 0; j < QI; ++j) {
    const int e = min(p * NT + tid + j * P * NT, Hq * HALF - 1);
    const int hq = e / HALF, i = e - hq * HALF;
    const int64_t qi = ((int64_t)b * Hq + hq) * D + i;
    q0v[j] = load_elem<BF16>(a.q, qi);
    q1v[j] = load_elem<BF16>(a.q, qi + HALF);
  }
  // keys of KV heads p + P wv, p + P (wv + 4), ...: the first one loaded now
  const int h0 = p + P * wv;
  float k0 = 0.0f, k1 = 0.0f;
  if (h0 < Hkv && lane < HALF) {
    k0 = load_elem<BF16>(a.k, (int64_t)(b * Hkv + h0) * D + lane);
    k1 = load_elem<BF16>(a.k, (int64_t)(b * Hkv + h0) * D + lane + HALF);
  }
  // ---- x W_dn and x W_dec over rows [p D / P, (p + 1) D / P), 128
  // threads each; the last wave forms the RoPE table of the position
  // meanwhile
  if (tid < NH) {
    gemv_partial<BF16, NH>(pn, tid, r0, r1, a.W_dn, xrow, s_red);
  } else if (tid < 2 * NH) {
    gemv_partial<BF16, NH>(pd, tid - NH, r0, r1, a.W_dec, xrow, s_red + NH);
  } else {
    const RopeTable rt{a.inv_freq, a.next_pos[b], HALF, s_cs, s_sn};
    for (int i = tid - 2 * NH; i < HALF; i += 64) rope_entry(rt, i);
  }
  __syncthreads();
  const int ZC = 3 * Hkv + a.r;
  if (tid < a.r) w.zdec[((int64_t)b * P + p) * ZC + 3 * Hkv + tid] = gemv_finish(pn, tid, s_red);
  if (tid < 3 * Hkv) w.zdec[((int64_t)b * P + p) * ZC + tid] = gemv_finish(pd, tid, s_red + NH);
  // ---- rotated queries
#pragma unroll
  for (int j = 0; j < QI; ++j) {
    const int e = p * NT + tid + j * P * NT;
    if (e < Hq * HALF) {
      const int hq = e / HALF, i = e - hq * HALF;
      const int64_t qi = ((int64_t)b * Hq + hq) * D + i;
      store_query<BF16>(w, qi, fmaf(q0v[j], s_cs[i], -q1v[j] * s_sn[i]));
      store_query<BF16>(w, qi + HALF, fmaf(q1v[j], s_cs[i], q0v[j] * s_sn[i]));
    }
  }
  for (int e = p * NT + tid + QI * P * NT; e < Hq * HALF; e += P * NT) {  // more than QI blocks
    const int hq = e / HALF, i = e - hq * HALF;
    const int64_t qi = ((int64_t)b * Hq + hq) * D + i;
    const float a0 = load_elem<BF16>(a.q, qi), a1 = load_elem<BF16>(a.q, qi + HALF);
    store_query<BF16>(w, qi, fmaf(a0, s_cs[i], -a1 * s_sn[i]));
    store_query<BF16>(w, qi + HALF, fmaf(a1, s_cs[i], a0 * s_sn[i]));
  }
  // ---- the stored keys (L2-normalised, rotated, rounded like the cache), one wave per head
  for (int h = h0; h < Hkv; h += P * (NT / 64)) {
    const int s = b * Hkv + h;
    if (h != h0 && lane < HALF) {
      k0 = load_elem<BF16>(a.k, (int64_t)s * D + lane);
      k1 = load_elem<BF16>(a.k, (int64_t)s * D + lane + HALF);
    }
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(k0 * k0 + k1 * k1)), 1e-12f);
    if (lane < HALF) {
      const float n0 = k0 * inv, n1 = k1 * inv;
      float rr0 = fmaf(n0, s_cs[lane], -n1 * s_sn[lane]);
      float rr1 = fmaf(n1, s_cs[lane], n0 * s_sn[lane]);
      if constexpr (BF16) {
        const uint16_t h0 = f32_to_bf16(rr0), h1 = f32_to_bf16(rr1);
        w.tkb[(int64_t)s * D + lane] = h0;
        w.tkb[(int64_t)s * D + lane + HALF] = h1;
        rr0 = bf16_to_f32(h0);
        rr1 = bf16_to_f32(h1);
      }
      w.tkey[(int64_t)s * D + lane] = rr0;
      w.tkey[(int64_t)s * D + lane + HALF] = rr1;
    }
  }
}

// Column col of z = x [W_dec | W_dn] of sequence b (the P row-slice partials
// added), and log sigmoid(z + b_dec) of a gate column
__device__ __forceinline__ float token_z(const LayerArgs& a, const DecodeWs& w, int b, int col) {
  const int ZC = 3 * a.H_kv + a.r;
  float z = 0.0f;
#pragma unroll
  for (int p = 0; p < kTokParts; ++p) z += w.zdec[((int64_t)b * kTokParts + p) * ZC + col];
  return z;
}
__device__ __forceinline__ float token_gate(const LayerArgs& a, const DecodeWs& w, int b, int col) {
  return log_sigmoid(token_z(a, w, b, col) + a.b_dec[col]);
}

// ---------------------------------------------------------------------------
// launch 2: the tiles
// ---------------------------------------------------------------------------
// Wait encodings (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): everything outstanding, or only the LDS/scalar counter.
constexpr int kWaitAll = 0;
constexpr int kWaitLgkm = 0xC07F;  // vmcnt 63, expcnt 7, lgkmcnt 0

// A tile's record and what follows from it.
struct TileInfo {
  int seg, len, ntile, pbase, kt, b, h;
  int64_t off;
  bool single;
};

__device__ __forceinline__ TileInfo tile_info(const int4& m0, const int4& m1, int Hkv) {
  TileInfo t;
  t.seg = m0.x;
  t.kt = m0.y;
  t.len = m0.z;
  t.ntile = m0.w;
  t.pbase = m1.x;  // record number of the segment's first tile
  t.off = (int64_t)(uint32_t)m1.y | ((int64_t)m1.z << 32);
  t.single = t.ntile == 1;
  t.b = t.seg / Hkv;
  t.h = t.seg - t.b * Hkv;
  return t;
}

// LDS of the part both tile kernels share.
template <int D, int G>
struct TailLds {
  float pm[kTileWaves * G], pl[kTileWaves * G];  // wave partials: max (log2 units), sum
  float po[kTileWaves * G * D];                  // wave partials: weighted V
  float es[G];                                   // the token's own logits (log2 units)
  float u[kMaxRank];                             // u = x W_dn
  int cnt[kTileWaves];                           // live entries per wave
  int kt, pre, flag;
};

template <int D, int G>
constexpr int tail_opt() {  // outputs (g, i) per thread
  return (G * D + kTileThreads - 1) / kTileThreads;
}

// After the wave partials and live counts are in LDS: the tile's partial per
// output (g, i) in registers; for a segment of several tiles the partial is
// published and marks the tile that merges them (L.flag).  Without COMPACT
// that is the tile that arrives last (an arrival counter).  With COMPACT the
// live count (the first tile's is its inclusive prefix) is published once the
// partial is visible, the look-back over the earlier tiles of the segment
// gives the survivors' destination (L.pre), and the segment's last tile
// merges: its look-back sees every earlier tile's count, so their partials
// are visible too.  Ends with a barrier.
template <int D, int G, bool COMPACT>
__device__ __forceinline__ void tile_publish(const DecodeKArgs& K, const TileInfo& t, TailLds<D, G>& L, int count,
                                             float* Mo, float* Lo, float* Oo) {
  constexpr int NT = kTileThreads, OPT = tail_opt<D, G>();
  const DecodeWs& w = K.w;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = min(u * NT + tid, G * D - 1);
    const int g = idx / D;
    const int i = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w2 = 0; w2 < kTileWaves; ++w2) M = fmaxf(M, L.pm[w2 * G + g]);
    const float Ms = (M == kNegInf) ? 0.0f : M;
    float Ls = 0.0f, O = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kTileWaves; ++w2) {
      const float wgt = __builtin_amdgcn_exp2f(L.pm[w2 * G + g] - Ms);
      Ls = fmaf(L.pl[w2 * G + g], wgt, Ls);
      O = fmaf(L.po[(w2 * G + g) * D + i], wgt, O);
    }
    Mo[u] = M;
    Lo[u] = Ls;
    Oo[u] = O;
  }
  if (!t.single) {
    const int64_t prow = (int64_t)(t.pbase + t.kt);
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = u * NT + tid;
      if (idx < G * D) {
        const int g = idx / D;
        const int i = idx - g * D;
        st_coh(w.part_o + (prow * G + g) * D + i, Oo[u]);
        if (i == 0) {
          st_coh(w.part_ml + (prow * G + g) * 2 + 0, Mo[u]);
          st_coh(w.part_ml + (prow * G + g) * 2 + 1, Lo[u]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    if constexpr (COMPACT) {
      if (tid == 0) {
        st64_coh(&K.ctl.dec_state[prow], (unsigned long long)((count << 2) | (t.kt == 0 ? 2 : 1)));
        L.flag = t.kt == t.ntile - 1;
      }
    } else {
      if (tid == 0) L.flag = (add_coh(&w.cnt[t.seg], 1) == t.ntile - 1);
    }
  }
  if (!COMPACT || t.single || t.kt == 0) {
    if (tid == 0) L.pre = 0;
  } else if (wv == 0) {
    const unsigned long long* st = K.ctl.dec_state + t.pbase;
    int prefix = 0;
    int cpos = t.kt - 1;  // next predecessor to examine
    int spins = 0;
    while (true) {
      const int pc2 = cpos - lane;  // lane l reads predecessor cpos - l
      const unsigned long long sv = (pc2 >= 0) ? ld64_coh(&st[pc2]) : 0ull;
      const int flag = (pc2 < 0) ? 2 : (int)(sv & 3u);  // tile -1 acts as prefix 0
      const int val = (pc2 < 0) ? 0 : (int)((uint32_t)sv >> 2);
      const uint64_t inc = __ballot(flag == 2);
      const uint64_t none = __ballot(flag == 0);
      const int stop = inc ? (int)__builtin_ctzll(inc) : 64;
      const uint64_t need = (stop >= 63) ? ~0ull : ((2ull << stop) - 1);
      if ((none & need) == 0) {
        prefix += wave_isum((lane <= stop) ? val : 0);
        if (stop < 64) break;
        cpos -= 64;
        continue;
      }
      if (++spins > kSpinLimitDec) {
        if (lane == 0) atomicOr(K.a.status, 2);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      st64_coh(&K.ctl.dec_state[t.pbase + t.kt], (unsigned long long)(((prefix + count) << 2) | 2));
      L.pre = prefix;
    }
  }
  __syncthreads();
}

// The output gate's weights of this thread's outputs (g, i): the first kUp
// rows of W_up's column and b_up.  A tile that will merge can load them when
// it starts (they are usually cold in HBM), long before the merge needs them.
template <int D, int G, bool BF16>
struct GateUp {
  static constexpr int kUp = 16;
  static constexpr int OPT = tail_opt<D, G>();
  static constexpr int UPF = OPT <= 2 ? OPT : 0;  // outputs whose W_up column is held in registers
  float wup[UPF > 0 ? UPF : 1][kUp];
  float bup[OPT];
  __device__ __forceinline__ void load(const LayerArgs& a, int h) {
    const int Hq = a.H_q;
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = min(u * kTileThreads + (int)threadIdx.x, G * D - 1);
      const int col = (h * G) * D + idx;
      bup[u] = a.b_up ? a.b_up[col] : 0.0f;
      if (u < UPF) {
#pragma unroll
        for (int q = 0; q < kUp; ++q) wup[u][q] = load_elem<BF16>(a.W_up, (int64_t)min(q, a.r - 1) * Hq * D + col);
      }
    }
  }
};

// The segment's output (by the tile that merges: every tile's partial, this
// one's in registers when it is the only one, the token's own term, the
// output gate), then the new entry and the new length (by the segment's last
// tile when compacting, else by the merging tile).  Every load the merge
// needs (the first TC tiles' partials, the token's value, u, W_up, the rotated
// query and key) is issued before any is used, so a merge of up to TC tiles
// waits on memory once.
template <int D, int G, bool BF16, bool COMPACT, int TC0>
__device__ __forceinline__ void tile_finish(const DecodeKArgs& K, const TileInfo& t, TailLds<D, G>& L, bool combines,
                                            int npos, float* Mo, float* Lo, float* Oo, GateUp<D, G, BF16>& gu,
                                            bool gu_loaded) {
  constexpr int NT = kTileThreads, OPT = tail_opt<D, G>();
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int TC = TC0 / OPT > 2 ? TC0 / OPT : 2;  // tiles whose partials are loaded together
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int Hkv = a.H_kv, Hq = a.H_q;
  const int seg = t.seg, b = t.b, h = t.h;
  if (combines) {
    // the partials (max, sum, weighted V) of tiles p0 .. p0 + TC - 1 for this
    // thread's outputs (indices past the last tile reload it; they are skipped)
    float xm[TC][OPT], xl[TC][OPT], xo[TC][OPT];
    auto load_pass = [&](int p0) {
#pragma unroll
      for (int p = 0; p < TC; ++p) {
        const int64_t tp = t.pbase + min(p0 + p, t.ntile - 1);
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
          const int idx = min(u * NT + tid, G * D - 1);
          const int g = idx / D;
          xo[p][u] = ld_coh(w.part_o + (tp * G + g) * D + (idx - g * D));
          xm[p][u] = ld_coh(w.part_ml + (tp * G + g) * 2 + 0);
          xl[p][u] = ld_coh(w.part_ml + (tp * G + g) * 2 + 1);
        }
      }
    };
    float M[OPT], Ls[OPT], O[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      M[u] = kNegInf;
      Ls[u] = 0.0f;
      O[u] = 0.0f;
    }
    auto merge_pass = [&](int p0) {
      const int tn = min(TC, t.ntile - p0);
#pragma unroll
      for (int u = 0; u < OPT; ++u) {
        float Mn = M[u];
#pragma unroll
        for (int p = 0; p < TC; ++p) Mn = (p < tn) ? fmaxf(Mn, xm[p][u]) : Mn;
        const float Ms = (Mn == kNegInf) ? 0.0f : Mn;
        const float rs = __builtin_amdgcn_exp2f(M[u] - Ms);
        float l = Ls[u] * rs, o = O[u] * rs;
#pragma unroll
        for (int p = 0; p < TC; ++p) {
          if (p < tn) {
            const float wgt = __builtin_amdgcn_exp2f(xm[p][u] - Ms);
            l = fmaf(xl[p][u], wgt, l);
            o = fmaf(xo[p][u], wgt, o);
          }
        }
        M[u] = Mn;
        Ls[u] = l;
        O[u] = o;
      }
    };
    if (!t.single) load_pass(0);
    // what the merge needs of the token: its value, u = x W_dn (the partials
    // added, into LDS), the output gate's weights (unless loaded already), and
    // its logit against its own key per head (wave 0, from the fp32 rotated
    // query and key)
    constexpr int kUp = GateUp<D, G, BF16>::kUp;
    constexpr int UPF = GateUp<D, G, BF16>::UPF;
    float vnv[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = min(u * NT + tid, G * D - 1);
      vnv[u] = elem_at<BF16>(reinterpret_cast<const char*>(a.v), (uint32_t)((seg * D + idx % D) * EB));
    }
    if (!gu_loaded) gu.load(a, h);
    if (tid < a.r) L.u[tid] = token_z(a, w, b, 3 * Hkv + tid);
    if (wv == 0) {
      const float qs2 = a.scale * kLog2e;
      const float* kt = w.tkey + (int64_t)seg * D;
      float e[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float* qt = w.tq + ((int64_t)b * Hq + h * G + g) * D;
        e[g] = 0.0f;
#pragma unroll
        for (int i = lane; i < D; i += 64) e[g] = fmaf(qt[i], kt[i], e[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float eg = wave_sum(e[g]);
        if (lane == 0) L.es[g] = eg * qs2;
      }
    }
    if (!t.single) {
      merge_pass(0);
      for (int p0 = TC; p0 < t.ntile; p0 += TC) {
        load_pass(p0);
        merge_pass(p0);
      }
#pragma unroll
      for (int u = 0; u < OPT; ++u) {
        Mo[u] = M[u];
        Lo[u] = Ls[u];
        Oo[u] = O[u];
      }
    }
    __syncthreads();  // u and the token's logits
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = u * NT + tid;
      if (idx < G * D) {
        const int g = idx / D;
        const int col = (h * G) * D + idx;
        const float es = L.es[g];
        const float M = fmaxf(Mo[u], es);
        const float rs = __builtin_amdgcn_exp2f(Mo[u] - M);  // Mo = -inf gives 0
        const float pe = __builtin_amdgcn_exp2f(es - M);
        const float Lt = fmaf(Lo[u], rs, pe);
        const float O = fmaf(Oo[u], rs, pe * vnv[u]);
        float z = gu.bup[u];
        if (u < UPF) {
#pragma unroll
          for (int q = 0; q < kUp; ++q)
            if (q < a.r) z = fmaf(L.u[q], gu.wup[u < UPF ? u : 0][q], z);
        } else {
          for (int q = 0; q < min(a.r, kUp); ++q)
            z = fmaf(L.u[q], load_elem<BF16>(a.W_up, (int64_t)q * Hq * D + col), z);
        }
        for (int q = kUp; q < a.r; ++q) z = fmaf(L.u[q], load_elem<BF16>(a.W_up, (int64_t)q * Hq * D + col), z);
        const int64_t yo = (int64_t)b * Hq * D + col;
        const float yv = sigmoid(z) * (O / Lt);
        if (a.y_bf16) {
          reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16(yv);
        } else {
          reinterpret_cast<float*>(a.y)[yo] = yv;
        }
      }
    }
  }
  const bool last = t.kt == t.ntile - 1;
  if (COMPACT ? last : combines) {
    const bool room = t.len < a.seg_cap[seg];
    if (room && tid < D) {
      const int64_t dst = (t.off + npos) * D + tid;
      const float kv = w.tkey[(int64_t)seg * D + tid];
      const float vv = elem_at<BF16>(reinterpret_cast<const char*>(a.v), (uint32_t)((seg * D + tid) * EB));
      if constexpr (BF16) {
        reinterpret_cast<uint16_t*>(a.K)[dst] = f32_to_bf16(kv);  // exact: kv is bf16-rounded
        reinterpret_cast<uint16_t*>(a.V)[dst] = f32_to_bf16(vv);  // exact: a bf16 input
      } else {
        reinterpret_cast<float*>(a.K)[dst] = kv;
        reinterpret_cast<float*>(a.V)[dst] = vv;
      }
    }
    if (tid == 0) {
      if (room) {
        a.lam[t.off + npos] = 0.0f;
        a.lk[t.off + npos] = token_gate(a, w, b, Hkv + h);
        if (COMPACT && K.kept) K.kept[t.off + npos] = t.len;
      } else {
        atomicOr(a.status, 1);
      }
      a.seg_len[seg] = room ? npos + 1 : npos;
      if (h == 0) a.next_pos[b] += 1;  // once per sequence; no tile reads it
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 caches: the dot products on the vector ALUs
// ---------------------------------------------------------------------------
// Load the V rows of a wave's entries straight into LDS at dst: for entry
// slot bb, each lane's 16-byte pieces (a lane reads back exactly what it
// loaded).
template <int D, int NB, bool BF16>
__device__ __forceinline__ void stage_v(const char* vseg, int f0, int relmax, int c, u32x4* dst) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int RP = BF16 ? 1 : 2;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int rel = min(f0 + bb, relmax);
    const uint32_t ro = (uint32_t)(rel * D + 8 * c) * EB;
#pragma unroll
    for (int pp = 0; pp < RP; ++pp)
      __builtin_amdgcn_global_load_lds(vseg + ro + 16 * pp, to_lds(dst + (bb * RP + pp) * 64), 16, 0, 0);
  }
}

template <int D, int G, bool BF16, bool COMPACT>
__global__ __launch_bounds__(kTileThreads, 3) void decode_tile_kernel(DecodeKArgs karg) {
  const DecodeKArgs& K = *(const DecodeKArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  using Sh = TileShape<D, decode_nb(D, G)>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, TWG = Sh::TWG;
  constexpr int OPT = tail_opt<D, G>();
  constexpr int EB = BF16 ? 2 : 4;  // bytes per element
  constexpr int RP = BF16 ? 1 : 2;  // 16-byte pieces of a lane's 8 elements
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane / LPE;
  const int c = lane - grp * LPE;
  const int Hkv = a.H_kv;
  const int Hq = a.H_q;

  __shared__ TailLds<D, G> L;
  __shared__ float s_tp[kTileWaves][NGW * D];     // per-wave transpose of the weighted V
  __shared__ u32x4 s_v[kTileWaves][NB * RP][64];  // the wave's V rows (loaded straight into LDS)

  // One workgroup per tile.  The tile number within its segment comes from a
  // per-segment ticket, so a tile's predecessors in its segment are held by
  // workgroups that started earlier and every wait below ends.  The record's
  // own number (the ticket's value when workgroups start in order) is used
  // to start the loads at once; another ticket value reloads.
  const int tile = blockIdx.x;
  const int4 m0 = w.map[2 * tile + 0];  // read with the tile count (a record past it is never used)
  const int4 m1 = w.map[2 * tile + 1];
  if (tile >= *w.ntiles) return;
  TileInfo t = tile_info(m0, m1, Hkv);
  const int len = t.len;
  const int b = t.b, h = t.h, seg = t.seg;
  char* const Kseg = reinterpret_cast<char*>(a.K) + t.off * (D * EB);
  char* const Vseg = reinterpret_cast<char*>(a.V) + t.off * (D * EB);
  const char* const lamseg = reinterpret_cast<const char*>(a.lam + t.off);
  const char* const lkseg = reinterpret_cast<const char*>(a.lk + t.off);
  const int relmax = max(len - 1, 0);
  if (!t.single && tid == 0) L.kt = add_coh(&w.segtk[seg], 1);

  // ---- cached entries: every load issued first, from the segment's base
  // with 32-bit offsets; slots past the end read the last entry (masked below)
  Row8<BF16> kr[NB];
  float lamv[NB], lkv[NB];
  auto load_rows = [&](int k) {
    const int f0 = k * TWG + wv * TW + grp * NB;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int rel = min(f0 + bb, relmax);
      const uint32_t ro = (uint32_t)(rel * D + 8 * c) * EB;
      row_load_at<BF16>(kr[bb], Kseg, ro);
      lamv[bb] = ld_at<float>(lamseg, (uint32_t)rel * 4);
      lkv[bb] = ld_at<float>(lkseg, (uint32_t)rel * 4);
    }
  };
  load_rows(t.kt);
  // ---- the token: rotated queries of the group and the stored key (8 dims
  // per lane), the query/similarity part of the pair term
  float qv[G][8], ktv[8];
  {
    const float* qrow = w.tq + ((int64_t)b * Hq + h * G) * D + 8 * c;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float4 x0 = *reinterpret_cast<const float4*>(qrow + g * D);
      const float4 x1 = *reinterpret_cast<const float4*>(qrow + g * D + 4);
      qv[g][0] = x0.x; qv[g][1] = x0.y; qv[g][2] = x0.z; qv[g][3] = x0.w;
      qv[g][4] = x1.x; qv[g][5] = x1.y; qv[g][6] = x1.z; qv[g][7] = x1.w;
    }
    const float* krow = w.tkey + (int64_t)seg * D + 8 * c;
    const float4 x0 = *reinterpret_cast<const float4*>(krow);
    const float4 x1 = *reinterpret_cast<const float4*>(krow + 4);
    ktv[0] = x0.x; ktv[1] = x0.y; ktv[2] = x0.z; ktv[3] = x0.w;
    ktv[4] = x1.x; ktv[5] = x1.y; ktv[6] = x1.z; ktv[7] = x1.w;
  }
  const PairCoef pc = pair_coef(a.terms);
  const float lq = (a.terms & 1) ? token_gate(a, w, b, h) : 0.0f;
  const float lbt = (a.terms & 4) ? token_gate(a, w, b, 2 * Hkv + h) : 0.0f;
  const float row2 = (lq + lbt) * pc.inv_n2;
  if (!t.single) {
    __syncthreads();
    if (L.kt != t.kt) {  // started out of order: this workgroup takes the ticket's tile
      t.kt = L.kt;
      load_rows(t.kt);
    }
  }
  const int e0 = t.kt * TWG + wv * TW + grp * NB;
  // the V rows, needed after the logits: straight into LDS, no registers held
  stage_v<D, NB, BF16>(Vseg, e0, relmax, c, &s_v[wv][0][0]);

  const float tau = K.tau;
  const float qs2 = a.scale * kLog2e;
  const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;

  // ---- dot products, pair term, bias update, logits
  float e2[G][NB];
  float newlam[NB];
  bool live[NB], changed[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const bool valid = e0 + bb < len;
    row_zero_if<BF16>(kr[bb], !valid);  // slots past the end may hold anything
    float kf[8];
    row_f32<BF16>(kr[bb], kf);
    float ps = 0.0f;
    float pq[G];
#pragma unroll
    for (int g = 0; g < G; ++g) pq[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ps = fmaf(ktv[i], kf[i], ps);
#pragma unroll
      for (int g = 0; g < G; ++g) pq[g] = fmaf(qv[g][i], kf[i], pq[g]);
    }
    ps = group_sum<LPE>(ps);
#pragma unroll
    for (int g = 0; g < G; ++g) pq[g] = group_sum<LPE>(pq[g]);
    const float l0 = valid ? lamv[bb] : kNegInf;
    const bool alive = valid && (l0 >= tau);
    const float A = pair_A(pc, row2, lkv[bb] * kscale, ps);
    const float l1 = alive ? l0 + A : l0;
    live[bb] = alive && (l1 >= tau);
    newlam[bb] = l1;
    changed[bb] = alive;
    const float lb2 = l1 * kLog2e;
#pragma unroll
    for (int g = 0; g < G; ++g) e2[g][bb] = live[bb] ? fmaf(pq[g], qs2, lb2) : kNegInf;
  }

  // ---- this tile's live entries (compaction): lane grp * LPE + bb owns
  // entry bb of its group; entries in tile order are (wave, group, entry)
  uint64_t mask = 0;
  if constexpr (COMPACT) {
    bool mine_live = false;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) mine_live = (c == bb) ? live[bb] : mine_live;
    mask = __ballot(c < NB && mine_live);
    if (lane == 0) L.cnt[wv] = __popcll(mask);
  }

  // ---- wave partial per head: max over the wave first, then sums relative to it
  float ms[G], lw[G], o8[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = e2[g][0];
#pragma unroll
    for (int bb = 1; bb < NB; ++bb) m = fmaxf(m, e2[g][bb]);
    ms[g] = across_groups_max<LPE>(m);
    lw[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o8[g][i] = 0.0f;
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);  // the V rows are in LDS
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    float vf[8];
    Row8<BF16> vrow;
#pragma unroll
    for (int pp = 0; pp < RP; ++pp) vrow.w[pp] = s_v[wv][bb * RP + pp][lane];
    row_zero_if<BF16>(vrow, e0 + bb >= len);  // slots past the end may hold anything
    row_f32<BF16>(vrow, vf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = __builtin_amdgcn_exp2f(e2[g][bb] - ((ms[g] == kNegInf) ? 0.0f : ms[g]));
      lw[g] += p;
#pragma unroll
      for (int i = 0; i < 8; ++i) o8[g][i] = fmaf(p, vf[i], o8[g][i]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = across_groups_sum<LPE>(lw[g]);
    // the groups' weighted V summed through a per-wave LDS transpose: each
    // lane writes its 8 sums, then lane j adds dimension j (and j + 64) over
    // the groups.  LDS operations of one wave complete in order.
    float* tp = s_tp[wv];  // [group][D]
    {
      float4* dst = reinterpret_cast<float4*>(tp + grp * D + 8 * c);
      dst[0] = make_float4(o8[g][0], o8[g][1], o8[g][2], o8[g][3]);
      dst[1] = make_float4(o8[g][4], o8[g][5], o8[g][6], o8[g][7]);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int half = 0; half < D / 64; ++half) {
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < NGW; ++q) sum += tp[q * D + half * 64 + lane];
      L.po[(wv * G + g) * D + half * 64 + lane] = sum;
    }
    __builtin_amdgcn_wave_barrier();  // the next head reuses the scratch
    if (lane == 0) {
      L.pm[wv * G + g] = ms[g];
      L.pl[wv * G + g] = l;
    }
  }
  __syncthreads();  // partials and live counts in LDS

  int count = 0, wbase = 0;
  if constexpr (COMPACT) {
#pragma unroll
    for (int w2 = 0; w2 < kTileWaves; ++w2) {
      wbase += (w2 < wv) ? L.cnt[w2] : 0;
      count += L.cnt[w2];
    }
  } else {
    if (c < NB) {  // lane c of a group stores entry c's bias
      float val = newlam[0];
      bool ch = changed[0];
#pragma unroll
      for (int bb = 1; bb < NB; ++bb) {
        val = (c == bb) ? newlam[bb] : val;
        ch = (c == bb) ? changed[bb] : ch;
      }
      if (ch) a.lam[t.off + e0 + c] = val;
    }
  }

  float Mo[OPT], Lo[OPT], Oo[OPT];
  tile_publish<D, G, COMPACT>(K, t, L, count, Mo, Lo, Oo);
  const bool combines = t.single || L.flag;

  int npos = len;  // where the new entry goes
  if constexpr (COMPACT) {
    // ---- the survivors, in order; rows already in place are not rewritten
    const int P = L.pre;
    int32_t* const kept = K.kept;
    const int myrank =
        wbase + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int rk = __shfl(myrank, grp * LPE + bb, 64);
      if (live[bb]) {
        const int rel = P + rk;
        const int64_t dst = t.off + rel;
        const bool moves = rel != e0 + bb;
        if (moves) {
          const uint32_t ro = (uint32_t)(rel * D + 8 * c) * EB;
          row_store_at<BF16>(kr[bb], Kseg, ro);
          Row8<BF16> vrow;
#pragma unroll
          for (int pp = 0; pp < RP; ++pp) vrow.w[pp] = s_v[wv][bb * RP + pp][lane];
          row_store_at<BF16>(vrow, Vseg, ro);
        }
        if (c == bb) {
          a.lam[dst] = newlam[bb];
          if (moves) a.lk[dst] = lkv[bb];
          if (kept) kept[dst] = e0 + bb;
        }
      }
    }
    npos = P + count;
  }
  GateUp<D, G, BF16> gu;
  tile_finish<D, G, BF16, COMPACT, 4>(K, t, L, combines, npos, Mo, Lo, Oo, gu, false);
}

// ---------------------------------------------------------------------------
// bf16 caches: the dot products on the matrix cores
// ---------------------------------------------------------------------------
// A wave takes TW entries (8 KB of keys and 8 KB of values).  The q.k
// products of 16 entries are one 16 x 16 tile S^T = K [q | k~]^T over the
// head dimension in 32-wide steps: row e of the tile is entry e, column j <
// G is query head j of the group (the rotated query as the sum of a high and
// a low bf16 part, two products into one accumulator, so the logit keeps
// about 16 bits of the fp32 query), column G is the token's stored key (the
// similarity).  Lane l holds rows 4 (l >> 4) .. + 3 of column l & 15, which
// is exactly the A operand layout of P V with P as heads x entries: k index
// 8 q + i of lane group q is entry 4 q + i of the first 16-entry block (i <
// 4) and entry 16 + 4 q + i - 4 of the second.  V comes through LDS, where
// the B operand (8 entries of one dimension per lane) is read as bf16
// halves.  The bias arithmetic runs once per entry, lane e of the wave
// holding entry e.
template <int D>
struct MfShape {
  static constexpr int TW = 4096 / D;   // entries per wave: 64 (d = 64) or 32 (d = 128)
  static constexpr int NBLK = TW / 16;  // 16-entry blocks of the q.k products
  static constexpr int KS = D / 32;     // 32-dim steps of the q.k products
  static constexpr int PS = TW / 32;    // 32-entry steps of the P V products
  static constexpr int NBD = D / 16;    // 16-dim blocks of the output
  static constexpr int TWG = TW * kTileWaves;
  static constexpr int RB = 2 * D;             // bytes per row
  static constexpr int RPI = 1024 / RB;        // V rows per staging load (64 lanes x 16 bytes)
  static constexpr int NI = TW / RPI;          // staging loads per wave
  static constexpr int VSTR = 1024 + 2048 / D;  // bytes between staged blocks (padding spreads the
                                                // B-operand reads over the LDS banks)
};

template <int D, int G, bool COMPACT>
__global__ __launch_bounds__(kTileThreads, 3) void decode_tile_mf_kernel(DecodeKArgs karg) {
  const DecodeKArgs& K = *(const DecodeKArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  using Sh = MfShape<D>;
  constexpr int TW = Sh::TW, NBLK = Sh::NBLK, KS = Sh::KS, PS = Sh::PS, NBD = Sh::NBD, TWG = Sh::TWG;
  constexpr int RB = Sh::RB, RPI = Sh::RPI, NI = Sh::NI, VSTR = Sh::VSTR;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int OPT = tail_opt<D, G>();
  static_assert(G < 16, "the similarity column follows the query columns");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, c16 = lane & 15;
  const int Hkv = a.H_kv;
  const int Hq = a.H_q;

  __shared__ TailLds<D, G> L;
  __shared__ __attribute__((aligned(16))) char s_v[kTileWaves][NI * VSTR];  // staged V rows
  __shared__ __attribute__((aligned(16))) float s_sim[kTileWaves][TW];       // similarity per entry
  __shared__ __attribute__((aligned(16))) float s_lb[kTileWaves][TW];        // bias (log2 units), -inf if out

  const int tile = blockIdx.x;
  const int4 m0 = w.map[2 * tile + 0];  // read with the tile count (a record past it is never used)
  const int4 m1 = w.map[2 * tile + 1];
  if (tile >= *w.ntiles) return;
  TileInfo t = tile_info(m0, m1, Hkv);
  // A tile waits only on earlier tiles of its segment.  A segment whose
  // records all lie among the first that fit on the GPU at once runs without
  // tickets: a tile takes its record's rows at once.  Otherwise the workgroups
  // of the segment take per-segment tickets: the one that arrives j-th takes
  // tile j, so it waits only on workgroups that started earlier.  (Loading the
  // record's rows first and again when the ticket differs read most rows
  // twice: tiles of one segment reach the ticket in no particular order.)
  const bool ticketed = m1.w != 0;
  const int len = t.len;
  const int b = t.b, h = t.h, seg = t.seg;
  char* const Kseg = reinterpret_cast<char*>(a.K) + t.off * RB;
  char* const Vseg = reinterpret_cast<char*>(a.V) + t.off * RB;
  const char* const lamseg = reinterpret_cast<const char*>(a.lam + t.off);
  const char* const lkseg = reinterpret_cast<const char*>(a.lk + t.off);
  const int relmax = max(len - 1, 0);
  if (ticketed && tid == 0) L.kt = add_coh(&w.segtk[seg], 1);

  // ---- cached entries, every load issued first: key rows as the A operand
  // (entry 16 blk + c16, dims 32 ks + 8 gq .. + 7), bias and key gate of
  // entry `lane`; slots past the end read the last entry
  u32x4 kb[NBLK][KS];
  float lamv, lkv;
  auto load_rows = [&](int k) {
    const int f0 = k * TWG + wv * TW;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const int rel = min(f0 + 16 * blk + c16, relmax);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb[blk][ks] = ld_at<u32x4>(Kseg, (uint32_t)(rel * RB + (32 * ks + 8 * gq) * 2));
    }
    const int rl = min(f0 + lane, relmax);
    lamv = ld_at<float>(lamseg, (uint32_t)rl * 4);
    lkv = ld_at<float>(lkseg, (uint32_t)rl * 4);
  };
  if (!ticketed) load_rows(t.kt);
  // ---- the token as the B operand: column c16 < G is query head h G + c16
  // (high and low bf16 parts), column G the stored key, the rest zero
  u32x4 qh[KS], ql[KS];
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool isq = c16 < G, isk = c16 == G;
    const int64_t qrow = ((int64_t)b * Hq + h * G + min(c16, G - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int dd = 32 * ks + 8 * gq;
      const u32x4 vh = *reinterpret_cast<const u32x4*>(w.tqh + qrow + dd);
      const u32x4 vl = *reinterpret_cast<const u32x4*>(w.tql + qrow + dd);
      const u32x4 vk = *reinterpret_cast<const u32x4*>(w.tkb + (int64_t)seg * D + dd);
      qh[ks] = isq ? vh : (isk ? vk : zero);
      ql[ks] = isq ? vl : zero;
    }
  }
  // a tile that merges (one-tile segment, or with COMPACT the segment's last
  // tile) loads the output gate's weights now, at head dim 64 (at 128 they
  // would cost occupancy); the merge needs them at the end
  GateUp<D, G, true> gu;
  const bool gu_early = D == 64 && (t.single || (COMPACT && t.kt == t.ntile - 1));
  if (gu_early) gu.load(a, h);
  const PairCoef pc = pair_coef(a.terms);
  const float lq = (a.terms & 1) ? token_gate(a, w, b, h) : 0.0f;
  const float lbt = (a.terms & 4) ? token_gate(a, w, b, 2 * Hkv + h) : 0.0f;
  const float row2 = (lq + lbt) * pc.inv_n2;
  if (ticketed) {
    __syncthreads();
    t.kt = L.kt;  // this workgroup takes the ticket's tile
    load_rows(t.kt);
  }
  const int e0 = t.kt * TWG + wv * TW;             // the wave's first entry
  const int nvalid = min(max(len - e0, 0), TW);  // wave-uniform
  char* const sv = s_v[wv];
  // the V rows, needed after the logits: straight into LDS (staging load i,
  // lane l: chunk l % CPR of entry RPI i + l / CPR)
  if (nvalid > 0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rel = min(e0 + RPI * i + lane / CPR, relmax);
      __builtin_amdgcn_global_load_lds(Vseg + (uint32_t)(rel * RB + (lane % CPR) * 16), to_lds(sv + i * VSTR), 16, 0,
                                       0);
    }
  }

  const float tau = K.tau;
  const float qs2 = a.scale * kLog2e;
  const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;
  float newlam = 0.0f;
  bool live = false, changed = false;
  if (nvalid > 0) {
    // ---- q.k and the similarity
    f32x4 acc[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma_bf16(kb[blk][ks], qh[ks], s);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma_bf16(kb[blk][ks], ql[ks], s);
      acc[blk] = s;
    }
    // the similarity of entry 16 blk + 4 gq + i (column G) to the entry's lane
    if (c16 == G) {
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
        *reinterpret_cast<float4*>(&s_sim[wv][16 * blk + 4 * gq]) =
            make_float4(acc[blk][0], acc[blk][1], acc[blk][2], acc[blk][3]);
    }
    __builtin_amdgcn_wave_barrier();  // LDS operations of one wave complete in order
    {
      // ---- pair term and bias update, once per entry
      const bool valid = lane < nvalid;
      const float sim = s_sim[wv][min(lane, TW - 1)];
      const float l0 = valid ? lamv : kNegInf;
      const bool alive = valid && (l0 >= tau);
      const float A = pair_A(pc, row2, lkv * kscale, sim);
      const float l1 = alive ? l0 + A : l0;
      live = alive && (l1 >= tau);
      newlam = l1;
      changed = alive;
      if (lane < TW) s_lb[wv][lane] = live ? l1 * kLog2e : kNegInf;
    }
    __builtin_amdgcn_wave_barrier();
    // ---- logits of head c16 for entries 16 blk + 4 gq + i; max and sum per head
    float e2[NBLK][4];
    float m = kNegInf;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const float4 lb = *reinterpret_cast<const float4*>(&s_lb[wv][16 * blk + 4 * gq]);
      const float lbv[4] = {lb.x, lb.y, lb.z, lb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e2[blk][i] = (c16 < G) ? fmaf(acc[blk][i], qs2, lbv[i]) : kNegInf;  // rows past the end: lb = -inf
        m = fmaxf(m, e2[blk][i]);
      }
    }
    m = across_groups_max<16>(m);
    const float msub = (m == kNegInf) ? 0.0f : m;
    float p[NBLK][4];
    float lsum = 0.0f;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[blk][i] = __builtin_amdgcn_exp2f(e2[blk][i] - msub);
        lsum += p[blk][i];
      }
    }
    lsum = across_groups_sum<16>(lsum);
    // ---- P V (P in high and low bf16 parts), V^T from LDS
    __builtin_amdgcn_s_waitcnt(kWaitAll);  // the V rows are in LDS
    f32x4 o[NBD];
#pragma unroll
    for (int nb = 0; nb < NBD; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      u32x4 ph, pl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = (j < 2) ? p[2 * ps][2 * j] : p[2 * ps + 1][2 * j - 4];
        const float x1 = (j < 2) ? p[2 * ps][2 * j + 1] : p[2 * ps + 1][2 * j - 3];
        const uint32_t hi = pack2_bf16(x0, x1);
        ph[j] = hi;
        pl[j] = pack2_bf16(x0 - bf16_lo(hi), x1 - bf16_hi(hi));
      }
      // the LDS offsets of the lane's 8 entries (k index order), row part
      int eo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 32 * ps + ((j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4);
        eo[j] = (e / RPI) * VSTR + (e % RPI) * RB;
      }
#pragma unroll
      for (int nb = 0; nb < NBD; ++nb) {
        const int dof = 2 * (16 * nb + c16);
        u32x4 vb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo16 = *reinterpret_cast<const uint16_t*>(sv + eo[2 * j] + dof);
          const uint32_t hi16 = *reinterpret_cast<const uint16_t*>(sv + eo[2 * j + 1] + dof);
          vb[j] = lo16 | (hi16 << 16);
        }
        o[nb] = mfma_bf16(ph, vb, o[nb]);
        o[nb] = mfma_bf16(pl, vb, o[nb]);
      }
    }
    // ---- wave partials: lane l holds heads 4 gq + i, dimension 16 nb + c16
#pragma unroll
    for (int nb = 0; nb < NBD; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * gq + i;
        if (g < G) L.po[(wv * G + g) * D + 16 * nb + c16] = o[nb][i];
      }
    }
    if (gq == 0 && c16 < G) {
      L.pm[wv * G + c16] = m;
      L.pl[wv * G + c16] = lsum;
    }
  } else {
    // a wave past the end of the segment: neutral partials
    for (int idx = lane; idx < G * D; idx += 64) L.po[wv * G * D + idx] = 0.0f;
    if (lane < G) {
      L.pm[wv * G + lane] = kNegInf;
      L.pl[wv * G + lane] = 0.0f;
    }
  }
  uint64_t mask = 0;
  if constexpr (COMPACT) {
    mask = __ballot(live);
    if (lane == 0) L.cnt[wv] = __popcll(mask);
  }
  __syncthreads();  // partials and live counts in LDS

  int count = 0, wbase = 0;
  if constexpr (COMPACT) {
#pragma unroll
    for (int w2 = 0; w2 < kTileWaves; ++w2) {
      wbase += (w2 < wv) ? L.cnt[w2] : 0;
      count += L.cnt[w2];
    }
  } else {
    if (changed) a.lam[t.off + e0 + lane] = newlam;
  }

  float Mo[OPT], Lo[OPT], Oo[OPT];
  tile_publish<D, G, COMPACT>(K, t, L, count, Mo, Lo, Oo);
  const bool combines = t.single || L.flag;

  int npos = len;  // where the new entry goes
  if constexpr (COMPACT) {
    // ---- the survivors, in order; rows already in place are not rewritten.
    // rank of entry e: (its rank among the tile's survivors) or -1, from lane e
    const int P = L.pre;
    const int myrank =
        wbase + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    const int rk_e = live ? myrank : -1;
    if (nvalid > 0) {
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {  // keys from registers
        const int e = 16 * blk + c16;
        const int rk = __shfl(rk_e, e, 64);
        if (rk >= 0 && P + rk != e0 + e) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<u32x4*>(Kseg + (uint32_t)((P + rk) * RB + (32 * ks + 8 * gq) * 2)) = kb[blk][ks];
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {  // values from LDS
        const int e = RPI * i + lane / CPR;
        const int rk = __shfl(rk_e, e, 64);
        if (rk >= 0 && P + rk != e0 + e) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(sv + i * VSTR + lane * 16);
          *reinterpret_cast<u32x4*>(Vseg + (uint32_t)((P + rk) * RB + (lane % CPR) * 16)) = v;
        }
      }
    }
    if (live) {
      const int64_t dst = t.off + P + myrank;
      a.lam[dst] = newlam;
      if (P + myrank != e0 + lane) a.lk[dst] = lkv;
      if (K.kept) K.kept[dst] = e0 + lane;
    }
    npos = P + count;
  }
  tile_finish<D, G, true, COMPACT, 16>(K, t, L, combines, npos, Mo, Lo, Oo, gu, gu_early);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int tile_entries(int d, int nb) { return (64 / (d / 8)) * nb * kTileWaves; }

// Entries per tile (sizes the per-tile workspace rows and flags).
int decode_tile_entries(int d, int g, bool bf16) {
  if (bf16) return d == 64 ? MfShape<64>::TWG : MfShape<128>::TWG;
  return tile_entries(d, decode_nb(d, g));
}

static int64_t decode_max_tiles(const LayerArgs& a, int twg) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  return a.total_slots / twg + S + 1;
}

// Scratch after the control block.
static size_t decode_layout(const LayerArgs& a, int twg, DecodeWs* w, char* base) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int G = a.H_q / a.H_kv;
  const int64_t mt = decode_max_tiles(a, twg);
  size_t n = 0;
  auto take = [&](size_t bytes) {
    char* q = base ? base + n : nullptr;
    n += align_up(bytes, 256);
    return q;
  };
  int* ntiles = reinterpret_cast<int*>(take(sizeof(int)));
  int* segtk = reinterpret_cast<int*>(take(sizeof(int) * S));
  int4* map = reinterpret_cast<int4*>(take(sizeof(int4) * 2 * mt));
  float* tq = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  float* tkey = reinterpret_cast<float*>(take(sizeof(float) * S * a.d));
  const size_t nh = a.bf16 ? 1 : 0;  // bf16 planes only for bf16 caches
  uint16_t* tqh = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * a.B * a.H_q * a.d * nh));
  uint16_t* tql = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * a.B * a.H_q * a.d * nh));
  uint16_t* tkb = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * S * a.d * nh));
  float* zdec = reinterpret_cast<float*>(take(sizeof(float) * a.B * kTokParts * (3 * a.H_kv + a.r)));
  float* part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  float* part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  if (w) {
    w->ntiles = ntiles;
    w->segtk = segtk;
    w->map = map;
    w->tq = tq;
    w->tkey = tkey;
    w->tqh = tqh;
    w->tql = tql;
    w->tkb = tkb;
    w->zdec = zdec;
    w->part_o = part_o;
    w->part_ml = part_ml;
    w->max_tiles = (int)mt;
  }
  return n;
}

size_t decode_ws_bytes(const LayerArgs& a, int twg) { return decode_layout(a, twg, nullptr, nullptr); }

DecodeWs decode_ws_carve(const LayerArgs& a, const Control& ctl, void* scratch, int twg) {
  DecodeWs w{};
  decode_layout(a, twg, &w, reinterpret_cast<char*>(scratch));
  w.cnt = ctl.dec_cnt;
  return w;
}

template <int D, int G, bool BF16>
static hipError_t launch_step(const LayerArgs& a, const DecodeWs& w, const Control& ctl, float tau, bool compact,
                              int32_t* kept, hipStream_t st) {
  const int twg = decode_tile_entries(D, G, BF16);
  DecodeKArgs k{a, w, ctl, tau, kept, twg, 0};
  const int64_t mt = decode_max_tiles(a, twg);
  if (mt > (1 << 30)) return hipErrorInvalidValue;
  if constexpr (BF16) {
    // the occupancy figure is the current device's; a stream of another
    // device runs every segment of several tiles with tickets (resident = 0)
    int cur = 0, sdev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return e;
    if (sdev == cur) {
      auto kern = compact ? decode_tile_mf_kernel<D, G, true> : decode_tile_mf_kernel<D, G, false>;
      e = resident_workgroups(kern, kTileThreads, &k.resident);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((decode_token_kernel<D, BF16>), dim3(a.B * kTokParts + 1), dim3(kTokThreads),
                     token_map_lds(a.B * a.H_kv, mt), st, k);
  const int grid = (int)mt;
  if constexpr (BF16) {
    auto kern = compact ? decode_tile_mf_kernel<D, G, true> : decode_tile_mf_kernel<D, G, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kTileThreads), 0, st, k);
  } else {
    if (compact) {
      hipLaunchKernelGGL((decode_tile_kernel<D, G, false, true>), dim3(grid), dim3(kTileThreads), 0, st, k);
    } else {
      hipLaunchKernelGGL((decode_tile_kernel<D, G, false, false>), dim3(grid), dim3(kTileThreads), 0, st, k);
    }
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_step_g(const LayerArgs& a, const DecodeWs& w, const Control& ctl, float tau, bool compact,
                                int32_t* kept, hipStream_t st) {
  switch (a.H_q / a.H_kv) {
    case 1: return launch_step<D, 1, BF16>(a, w, ctl, tau, compact, kept, st);
    case 2: return launch_step<D, 2, BF16>(a, w, ctl, tau, compact, kept, st);
    case 3: return launch_step<D, 3, BF16>(a, w, ctl, tau, compact, kept, st);
    case 4: return launch_step<D, 4, BF16>(a, w, ctl, tau, compact, kept, st);
    case 8: return launch_step<D, 8, BF16>(a, w, ctl, tau, compact, kept, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const LayerArgs& a, const DecodeWs& w, const Control& ctl, float tau, bool compact,
                         int32_t* kept, hipStream_t st) {
  if (a.d == 64) {
    return a.bf16 ? launch_step_g<64, true>(a, w, ctl, tau, compact, kept, st)
                  : launch_step_g<64, false>(a, w, ctl, tau, compact, kept, st);
  }
  return a.bf16 ? launch_step_g<128, true>(a, w, ctl, tau, compact, kept, st)
                : launch_step_g<128, false>(a, w, ctl, tau, compact, kept, st);
}

}  // namespace ua
