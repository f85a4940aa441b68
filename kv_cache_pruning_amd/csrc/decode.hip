// UA decode step on a ragged, per-KV-head pruned cache (gfx950), one launch,
// optionally with the in-place compaction of every segment in the same launch.
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
// Work items are numbered and handed out by an atomic ticket to a persistent
// grid (at most one workgroup per compute unit), so every wait below is on an
// item that a running workgroup already holds.
//  * items [0, B): per sequence, the gates log sigmoid(x W_dec + b_dec) of
//    every KV head (query, key and similarity columns); items [B, 2B): u =
//    x W_dn.  Results are published as 64-bit words whose high half is the
//    call's tag, so a reader checks each word on its own: no flag, no ordering
//    between words.  Tiles read their two gate words after their loads, by
//    which time the gate items (drawn first) have normally published.
//  * later items: one tile of TWG entries of one segment (segment = sequence
//    and KV head), numbered segment by segment from the lengths at the start
//    of the call.  A tile issues its cache loads together with what it needs
//    of the token (its G queries, the key, its two gate words), forms the
//    rotated queries and stored key itself,
//    and reads each entry once: the key row feeds the G query dot products
//    and the key-similarity dot product, the pair term updates the log-bias,
//    and an online-softmax partial (max, sum, weighted V) is formed per
//    group of lanes, merged across the wave through an LDS transpose and
//    across the waves in LDS.
//  * With COMPACT the surviving entries move down in place: a tile publishes
//    its live count once all its rows are in registers and looks back over
//    the earlier tiles of its segment for its destination (decoupled
//    look-back); the look-back cannot finish before every earlier tile has
//    published, which orders the stores after the loads they overwrite.  Only
//    rows that move are rewritten; every survivor's new log-bias is stored.
//    Without COMPACT the log-biases are updated in place.
//  * A segment held by one tile (the common case) combines at once from LDS.
//    Otherwise each tile writes its partial to the workspace and the last to
//    arrive merges them.  The combine adds the token's own term, forms the
//    output gate from u and its slice of W_up, writes y and appends the new
//    entry (after the survivors when compacting).
//  * A workgroup draws its next ticket while its current item finishes.
//    Drawing a ticket past the last item is its exit; the workgroup that draws the last
//    ticket waits until every workgroup has finished and commits the new
//    lengths and positions.
//
// Cross-workgroup data go through relaxed agent-scope atomics (coherent across
// the XCDs without cache-wide write-back or invalidation).

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ldi_coh(const int* p) {
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

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kSpinLimitDec = 1 << 22;
constexpr int kWaveK = kDecWaves - 1;  // the wave that forms the stored key

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
// query heads per KV head.  Four keeps every load of a tile in flight together
// without spilling at group sizes up to 4; two leaves the tiles' fixed costs
// (the combine, the per-tile partials) to dominate at large batches, eight
// spills.  At group size 8 and head dim 64, four spills and two is faster.
constexpr int decode_nb(int d, int g) { return (d == 64 && g >= 8) ? 2 : 4; }

template <int D, int NB_>
struct DecodeShape {
  static constexpr int LPE = D / 8;     // lanes per entry (8 elements each)
  static constexpr int NGW = 64 / LPE;  // entry groups per wave
  static constexpr int NB = NB_;        // entries per group
  static constexpr int TW = NGW * NB;   // entries per wave
  static constexpr int TWG = TW * kDecWaves;
  static_assert(NB <= LPE, "lane c < NB of a group holds entry c's flags");
};

__device__ __forceinline__ int tiles_of(int n, int twg) { return n <= 0 ? 1 : ceil_div(n, twg); }

__device__ __forceinline__ unsigned long long tag_word(float v, uint32_t tag) {
  return ((unsigned long long)tag << 32) | __float_as_uint(v);
}

// ---------------------------------------------------------------------------
// per-sequence items: the gates log sigmoid(x W_dec + b_dec) of every KV head
// (3 H_kv columns: query, key, similarity), or u = x W_dn (r columns).  Each
// result is published as a tagged word.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ void seq_item(const LayerArgs& a, const Control& ctl, int b, bool gates, uint32_t tag,
                         float (*s_red)[8]) {
  constexpr int CW = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int NT = kDecThreads;
  constexpr int KR = 16;  // rows per thread per pass, all loads in flight together
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int Dm = a.D_model;
  const int ncols = gates ? 3 * a.H_kv : a.r;
  const char* const mbase = reinterpret_cast<const char*>(gates ? a.W_dec : a.W_dn);
  const bool vec = ncols % CW == 0;
  const int nch = vec ? ncols / CW : ncols;  // column groups (16-byte chunks or single columns)
  int npow = 1;
  while (npow < nch) npow <<= 1;
  const int R = NT / npow;  // row subsets
  const int kc = tid & (npow - 1), rsub = tid / npow;
  const bool own = kc < nch;
  const int mc0 = own ? (vec ? kc * CW : kc) : 0;
  const char* const xrow = reinterpret_cast<const char*>(a.x) + (int64_t)b * Dm * (BF16 ? 2 : 4);
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.0f;
  for (int rb = rsub; rb < Dm; rb += KR * R) {
    float xr[KR];
    u32x4 raw[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const int row = min(rb + q * R, Dm - 1);
      xr[q] = elem_at<BF16>(xrow, (uint32_t)row * (BF16 ? 2 : 4));
      const uint32_t e = (uint32_t)(row * ncols + mc0) * (BF16 ? 2 : 4);
      if (vec) {
        raw[q] = ld_at<u32x4>(mbase, e);
      } else {
        raw[q] = u32x4{__float_as_uint(elem_at<BF16>(mbase, e)), 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const float xv = (own && rb + q * R < Dm) ? xr[q] : 0.0f;
      if (vec) {
#pragma unroll
        for (int t = 0; t < CW; ++t) acc[t] = fmaf(xv, chunk_elem<BF16>(raw[q], t), acc[t]);
      } else {
        acc[0] = fmaf(xv, __uint_as_float(raw[q][0]), acc[0]);
      }
    }
  }
  // partial sums: reduced over the row subsets inside a wave when a wave holds
  // every column group, else one slot per thread
  int reff;
  if (npow <= 64) {
    for (int o = npow; o < 64; o <<= 1) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] += __shfl_xor(acc[t], o, 64);
    }
    if (lane < npow) {
#pragma unroll
      for (int t = 0; t < 8; ++t) s_red[wv * npow + lane][t] = acc[t];
    }
    reff = kDecWaves;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) s_red[tid][t] = acc[t];
    reff = R;
  }
  __syncthreads();
  unsigned long long* uw = ctl.uw + (int64_t)b * kUWords;
  if (tid < ncols) {
    const int grp = vec ? tid / CW : tid;
    const int t = vec ? tid % CW : 0;
    float z = 0.0f;
    for (int rr = 0; rr < reff; ++rr) z += s_red[rr * npow + grp][t];
    if (gates) {
      st64_coh(uw + kMaxRank + tid, tag_word(log_sigmoid(z + a.b_dec[tid]), tag));
    } else {
      st64_coh(uw + tid, tag_word(z, tag));
    }
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// All kernel arguments in one struct, read through the kernel-argument
// segment pointer where they are used: passed as separate by-value
// parameters, every field is loaded at entry and most then spill from scalar
// registers into vector lanes, each use costing a VALU read.  The struct is
// the only explicit argument, so it starts the segment.
struct DecodeKArgs {
  LayerArgs a;
  DecodeWs w;
  Control ctl;
  float tau;
  int32_t* kept;
};

template <int D, int G, bool BF16, bool COMPACT>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(DecodeKArgs karg) {
  const DecodeKArgs& K = *(const DecodeKArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  const Control& ctl = K.ctl;
  const float tau = K.tau;
  int32_t* const kept = K.kept;
  using Sh = DecodeShape<D, decode_nb(D, G)>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, TWG = Sh::TWG;
  constexpr int NT = kDecThreads;
  constexpr int HALF = D / 2;
  constexpr int OPT = (G * D + NT - 1) / NT;  // outputs (g, i) per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.B * a.H_kv;
  const int Hkv = a.H_kv;
  const int Dm = a.D_model;
  const int r = a.r;

  __shared__ int s_id;
  __shared__ int s_scan[NT / 64 + 1];
  __shared__ int s_info[4];
  __shared__ int s_flag;
  __shared__ int s_pre;
  __shared__ int s_cnt[kDecWaves];
  __shared__ float s_red[NT][8];                              // per-sequence item: partial projections
  __shared__ float s_cs[HALF], s_sn[HALF];                    // RoPE table of the token's position
  __shared__ float s_tq[(G + 1) * D];                         // rotated queries of the group, then the stored key
  __shared__ float s_g[2];                                    // query and similarity gates (log sigmoid)
  __shared__ float s_po[kDecWaves * G * D];                   // wave partials: weighted V
  __shared__ float s_pm[kDecWaves * G], s_pl[kDecWaves * G];  // wave partials: max (log2), sum
  __shared__ float s_es[G];                                   // the token's own logits (log2 units)
  __shared__ float s_u[kMaxRank + 1];                         // u, then the new key's gate

  const uint32_t tag = (uint32_t)ctl.glob[kGlobSeq] + 1u;
  // Tickets are drawn by the first lane of the last wave (which loads no
  // lengths below) and kept in a register until the next item starts, so the
  // draw flies while the numbering or the current item runs.
  constexpr int kDrawer = NT - 64;
  int nxt = 0;
  if (tid == kDrawer) nxt = add_coh(&ctl.glob[kGlobTicket], 1);

  // Tile numbering from the segment lengths, done the first time a ticket
  // past the per-sequence items is drawn (the lengths stay unchanged until
  // the commit, which waits until every workgroup has finished).
  const int per = (S + NT - 1) / NT;
  const int sb = min(S, tid * per);
  const int se = min(S, sb + per);
  int mine = 0, excl = 0, total_items = 0;
  bool numbered = false;

  while (true) {
    if (tid == kDrawer) s_id = nxt;
    __syncthreads();
    const int id = s_id;

    if (id < 2 * a.B) {  // gate items first: tiles need them early
      seq_item<BF16>(a, ctl, id % a.B, id < a.B, tag, s_red);
      if (tid == kDrawer) nxt = add_coh(&ctl.glob[kGlobTicket], 1);
      continue;
    }
    if (!numbered) {
      for (int s = sb; s < se; ++s) mine += tiles_of(a.seg_len[s], TWG);
      int total_tiles;
      excl = block_exclusive_scan<NT>(mine, s_scan, &total_tiles);
      total_items = 2 * a.B + total_tiles;
      numbered = true;
    }

    if (id >= total_items) {
      // ---- exit.  Every workgroup reports that it has finished (its stores
      // done); the one that drew the last ticket waits for all of them and
      // commits lengths and positions.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) add_coh(&ctl.glob[kGlobDone], 1);
      if (id == total_items + (int)gridDim.x - 1) {
        if (tid == 0) {
          int spins = 0;
          while (ldi_coh(&ctl.glob[kGlobDone]) < (int)gridDim.x) {
            if (++spins > kSpinLimitDec) {
              atomicOr(a.status, 2);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        __syncthreads();
        for (int s = tid; s < S; s += NT) a.seg_len[s] = ldi_coh(&w.newlen[s]);
        for (int b = tid; b < a.B; b += NT) a.next_pos[b] += 1;
        if (tid == 0) {
          sti_coh(&ctl.glob[kGlobTicket], 0);
          sti_coh(&ctl.glob[kGlobDone], 0);
          sti_coh(&ctl.glob[kGlobSeq], (int)tag);
        }
      }
      break;
    }
    // ---- (segment, tile) of this item
    const int tix = id - 2 * a.B;
    if (tix >= excl && tix < excl + mine && per == 1) {
      s_info[0] = sb;
      s_info[1] = tix - excl;
      s_info[2] = mine;
      s_info[3] = excl;
    } else if (tix >= excl && tix < excl + mine) {
      int run = excl;
      for (int s = sb; s < se; ++s) {
        const int nt = tiles_of(a.seg_len[s], TWG);
        if (tix < run + nt) {
          s_info[0] = s;
          s_info[1] = tix - run;
          s_info[2] = nt;
          s_info[3] = run;
          break;
        }
        run += nt;
      }
    }
    __syncthreads();
    const int seg = s_info[0];
    const int kt_ = s_info[1];
    const int ntile = s_info[2];  // tiles of this segment
    const int pbase = s_info[3];  // tile number of its first tile
    const bool single = ntile == 1;
    const int b = seg / Hkv;
    const int h = seg - b * Hkv;
    const int len = a.seg_len[seg];
    const int cap = a.seg_cap[seg];
    const int64_t off = a.seg_off[seg];
    const float qs2 = a.scale * kLog2e;
    const int grp = lane / LPE;
    const int c = lane - grp * LPE;
    const int e0 = kt_ * TWG + wv * TW + grp * NB;

    // ---- cached entries: every load issued first, from the segment's base with
    // 32-bit offsets; slots past the end read the last entry (masked below)
    constexpr int EB = BF16 ? 2 : 4;  // bytes per element
    char* const Kseg = reinterpret_cast<char*>(a.K) + off * (D * EB);
    char* const Vseg = reinterpret_cast<char*>(a.V) + off * (D * EB);
    const char* const lamseg = reinterpret_cast<const char*>(a.lam + off);
    const char* const lkseg = reinterpret_cast<const char*>(a.lk + off);
    const int relmax = max(len - 1, 0);
    Row8<BF16> kr[NB], vr[NB];
    float lamv[NB], lkv[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int rel = min(e0 + bb, relmax);
      const uint32_t ro = (uint32_t)(rel * D + 8 * c) * EB;
      row_load_at<BF16>(kr[bb], Kseg, ro);
      row_load_at<BF16>(vr[bb], Vseg, ro);
      lamv[bb] = ld_at<float>(lamseg, (uint32_t)rel * 4);
      lkv[bb] = ld_at<float>(lkseg, (uint32_t)rel * 4);
    }
    // ---- the token: position, query pair (g, i) / (g, i + d/2), key pair, V
    const int pos = a.next_pos[b];
    const int qg = min(tid / HALF, G - 1), qi = tid % HALF;
    const char* const qrow = reinterpret_cast<const char*>(a.q);
    const uint32_t qb = (uint32_t)(((b * a.H_q + h * G + qg) * D + qi) * EB);
    const float q0 = elem_at<BF16>(qrow, qb);
    const float q1 = elem_at<BF16>(qrow, qb + HALF * EB);
    float k0 = 0.0f, k1 = 0.0f;
    if (wv == kWaveK && lane < HALF) {
      const uint32_t kb = (uint32_t)((seg * D + lane) * EB);
      k0 = elem_at<BF16>(reinterpret_cast<const char*>(a.k), kb);
      k1 = elem_at<BF16>(reinterpret_cast<const char*>(a.k), kb + HALF * EB);
    }
    float vn[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u)
      vn[u] = elem_at<BF16>(reinterpret_cast<const char*>(a.v), (uint32_t)((seg * D + (u * NT + tid) % D) * EB));
    // ---- the query and similarity gates from the sequence's gate item
    // (tagged words; checked, and re-read if stale, after the table)
    const unsigned long long* gword =
        ctl.uw + (int64_t)b * kUWords + kMaxRank + (tid == 0 ? h : 2 * Hkv + h);
    unsigned long long gwd = (tid < 2) ? ld64_coh(gword) : 0ull;
    // ---- RoPE table (fp64 angles) while the loads fly
    if (tid < HALF) {
      double sn, cs;
      sincos((double)pos * a.inv_freq[tid], &sn, &cs);
      s_cs[tid] = (float)cs;
      s_sn[tid] = (float)sn;
    }
    __syncthreads();
    // ---- rotated queries, the stored key (L2-normalised, rotated, rounded like the cache), gates
    if (tid < G * HALF) {
      s_tq[qg * D + qi] = fmaf(q0, s_cs[qi], -q1 * s_sn[qi]);
      s_tq[qg * D + qi + HALF] = fmaf(q1, s_cs[qi], q0 * s_sn[qi]);
    }
    if (wv == kWaveK) {
      const float inv = 1.0f / fmaxf(sqrtf(wave_sum(k0 * k0 + k1 * k1)), 1e-12f);
      if (lane < HALF) {
        const float n0 = k0 * inv, n1 = k1 * inv;
        float rr0 = fmaf(n0, s_cs[lane], -n1 * s_sn[lane]);
        float rr1 = fmaf(n1, s_cs[lane], n0 * s_sn[lane]);
        if constexpr (BF16) {
          rr0 = bf16_to_f32(f32_to_bf16(rr0));
          rr1 = bf16_to_f32(f32_to_bf16(rr1));
        }
        s_tq[G * D + lane] = rr0;
        s_tq[G * D + lane + HALF] = rr1;
      }
    }
    if (tid < 2) {
      int spins = 0;
      while ((uint32_t)(gwd >> 32) != tag) {
        if (++spins > kSpinLimitDec) {
          atomicOr(a.status, 2);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        gwd = ld64_coh(gword);
      }
      s_g[tid] = __uint_as_float((uint32_t)gwd);
    }
    __syncthreads();

    const PairCoef pc = pair_coef(a.terms);
    const float row2 = (((a.terms & 1) ? s_g[0] : 0.0f) + ((a.terms & 4) ? s_g[1] : 0.0f)) * pc.inv_n2;
    const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;
    float qv[G][8], ktv[8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[g][i] = s_tq[g * D + 8 * c + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) ktv[i] = s_tq[G * D + 8 * c + i];

    // ---- dot products, pair term, bias update, logits
    float e2[G][NB];
    float newlam[NB];
    bool live[NB], changed[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const bool valid = e0 + bb < len;
      row_zero_if<BF16>(kr[bb], !valid);  // slots past the end may hold anything
      row_zero_if<BF16>(vr[bb], !valid);
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
      if (lane == 0) s_cnt[wv] = __popcll(mask);
    }
    // ---- issued now, used by the combine: the sequence's tagged words (u, the
    // new key's gate)
    const unsigned long long* uword = ctl.uw + (int64_t)b * kUWords + (tid < r ? tid : kMaxRank + Hkv + h);
    unsigned long long uwd = (tid <= r) ? ld64_coh(uword) : 0ull;

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
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      float vf[8];
      row_f32<BF16>(vr[bb], vf);
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
      // the groups' weighted V summed through a per-wave LDS transpose (the
      // per-sequence item's scratch): each lane writes its 8 sums, then lane
      // j adds dimension j (and j + 64) over the groups.  LDS operations of
      // one wave complete in order, so no barrier is needed.
      float* tp = &s_red[wv * 64][0];  // [group][D]
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
        s_po[(wv * G + g) * D + half * 64 + lane] = sum;
      }
      __builtin_amdgcn_wave_barrier();  // the next head reuses the scratch
      if (lane == 0) {
        s_pm[wv * G + g] = ms[g];
        s_pl[wv * G + g] = l;
      }
    }
    // the output-gate weights of this thread's outputs, for the combine
    constexpr int kUp = 16;
    const int Hq = a.H_q;
    float up[OPT][kUp];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = min(u * NT + tid, G * D - 1);
      const int col = (h * G) * D + idx;
#pragma unroll
      for (int q = 0; q < kUp; ++q) up[u][q] = load_elem<BF16>(a.W_up, (int64_t)min(q, r - 1) * Hq * D + col);
    }
    // the next item, drawn while this one finishes (not earlier: workgroups
    // that start late must get their first items before early ones take a
    // second)
    if (tid == kDrawer) nxt = add_coh(&ctl.glob[kGlobTicket], 1);
    __syncthreads();  // partials and live counts in LDS; every row of the tile is in registers

    int count = 0, wbase = 0;
    if constexpr (COMPACT) {
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) {
        wbase += (w2 < wv) ? s_cnt[w2] : 0;
        count += s_cnt[w2];
      }
      // this tile's count (the first tile's is already its inclusive prefix)
      if (!single && tid == 0)
        st64_coh(&ctl.dec_state[pbase + kt_],
                 ((unsigned long long)tag << 32) | (uint32_t)((count << 2) | (kt_ == 0 ? 2 : 1)));
    } else {
      if (c < NB) {  // lane c of a group stores entry c's bias
        float val = newlam[0];
        bool ch = changed[0];
#pragma unroll
        for (int bb = 1; bb < NB; ++bb) {
          val = (c == bb) ? newlam[bb] : val;
          ch = (c == bb) ? changed[bb] : ch;
        }
        if (ch) a.lam[off + e0 + c] = val;
      }
    }

    // ---- the tile's partial per output (g, i): merge of the wave partials
    float Mo[OPT], Lo[OPT], Oo[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = min(u * NT + tid, G * D - 1);
      const int g = idx / D;
      const int i = idx - g * D;
      float M = kNegInf;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) M = fmaxf(M, s_pm[w2 * G + g]);
      const float Ms = (M == kNegInf) ? 0.0f : M;
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) {
        const float wgt = __builtin_amdgcn_exp2f(s_pm[w2 * G + g] - Ms);
        L = fmaf(s_pl[w2 * G + g], wgt, L);
        O = fmaf(s_po[(w2 * G + g) * D + i], wgt, O);
      }
      Mo[u] = M;
      Lo[u] = L;
      Oo[u] = O;
    }

    bool combines = single;
    if (!single) {
      // ---- publish the partial; the last tile of the segment to arrive merges
      const int64_t prow = (int64_t)(pbase + kt_);
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
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) s_flag = (add_coh(&w.cnt[seg], 1) == ntile - 1);
      __syncthreads();
      combines = s_flag;
      if (combines) {
        constexpr int TC = 8;  // tiles per pass, loads in flight together
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
          const int idx = min(u * NT + tid, G * D - 1);
          const int g = idx / D;
          const int i = idx - g * D;
          float M = kNegInf, L = 0.0f, O = 0.0f;
          for (int p0 = 0; p0 < ntile; p0 += TC) {
            float pm[TC], pl[TC], po[TC];
#pragma unroll
            for (int p = 0; p < TC; ++p) {
              const int64_t pr = (int64_t)(pbase + min(p0 + p, ntile - 1));
              pm[p] = ld_coh(w.part_ml + (pr * G + g) * 2 + 0);
              pl[p] = ld_coh(w.part_ml + (pr * G + g) * 2 + 1);
              po[p] = ld_coh(w.part_o + (pr * G + g) * D + i);
            }
            float Mn = M;
#pragma unroll
            for (int p = 0; p < TC; ++p) Mn = (p0 + p < ntile) ? fmaxf(Mn, pm[p]) : Mn;
            const float Ms = (Mn == kNegInf) ? 0.0f : Mn;
            const float rs = __builtin_amdgcn_exp2f(M - Ms);
            L *= rs;
            O *= rs;
#pragma unroll
            for (int p = 0; p < TC; ++p) {
              if (p0 + p < ntile) {
                const float wgt = __builtin_amdgcn_exp2f(pm[p] - Ms);
                L = fmaf(pl[p], wgt, L);
                O = fmaf(po[p], wgt, O);
              }
            }
            M = Mn;
          }
          Mo[u] = M;
          Lo[u] = L;
          Oo[u] = O;
        }
        if (tid == 0) sti_coh(&w.cnt[seg], 0);
      }
    }
    // the tile that appends the new entry: the combining one, or with
    // compaction the segment's last tile (it learns the final length)
    const bool appends = COMPACT ? (kt_ == ntile - 1) : combines;

    // ---- the sequence's tagged words, once they carry this call's tag
    if ((combines || appends) && tid <= r) {
      int spins = 0;
      while ((uint32_t)(uwd >> 32) != tag) {
        if (++spins > kSpinLimitDec) {
          atomicOr(a.status, 2);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        uwd = ld64_coh(uword);
      }
      s_u[tid] = __uint_as_float((uint32_t)uwd);
    }

    // ---- combine: the token's own term, the output gate, y
    if (combines) {
      if (wv < G) {  // the token's own logit per query head (one wave each)
        float e = 0.0f;
        for (int i = lane; i < D; i += 64) e = fmaf(s_tq[wv * D + i], s_tq[G * D + i], e);
        e = wave_sum(e);
        if (lane == 0) s_es[wv] = e * qs2;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < OPT; ++u) {
        const int idx = u * NT + tid;
        if (idx < G * D) {
          const int g = idx / D;
          const float es = s_es[g];
          const float M = fmaxf(Mo[u], es);
          const float rs = __builtin_amdgcn_exp2f(Mo[u] - M);  // Mo = -inf gives 0
          const float pe = __builtin_amdgcn_exp2f(es - M);
          const float L = fmaf(Lo[u], rs, pe);
          const float O = fmaf(Oo[u], rs, pe * vn[u]);
          const int col = (h * G) * D + idx;
          float z = a.b_up ? a.b_up[col] : 0.0f;
#pragma unroll
          for (int q = 0; q < kUp; ++q)
            if (q < r) z = fmaf(s_u[q], up[u][q], z);
          for (int q = kUp; q < r; ++q) z = fmaf(s_u[q], load_elem<BF16>(a.W_up, (int64_t)q * Hq * D + col), z);
          const int64_t yo = (int64_t)b * Hq * D + col;
          const float yv = sigmoid(z) * (O / L);
          if (a.y_bf16) {
            reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16(yv);
          } else {
            reinterpret_cast<float*>(a.y)[yo] = yv;
          }
        }
      }
    }

    int npos = len;  // where the new entry goes
    if constexpr (COMPACT) {
      // ---- destination of the survivors: look back over the earlier tiles
      if (single) {
        if (tid == 0) s_pre = 0;
      } else if (wv == 0 && kt_ == 0) {
        if (lane == 0) s_pre = 0;
      } else if (wv == 0) {
        const unsigned long long* st = ctl.dec_state + pbase;
        int prefix = 0;
        int cpos = kt_ - 1;  // next predecessor to examine
        int spins = 0;
        while (true) {
          const int pc2 = cpos - lane;  // lane l reads predecessor cpos - l
          const unsigned long long sv = (pc2 >= 0) ? ld64_coh(&st[pc2]) : 0ull;
          const bool cur = (pc2 < 0) || ((uint32_t)(sv >> 32) == tag);
          const int flag = (pc2 < 0) ? 2 : (cur ? (int)(sv & 3u) : 0);  // tile -1 acts as prefix 0
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
            if (lane == 0) atomicOr(a.status, 2);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) {
          st64_coh(&ctl.dec_state[pbase + kt_], ((unsigned long long)tag << 32) | (uint32_t)(((prefix + count) << 2) | 2));
          s_pre = prefix;
        }
      }
      __syncthreads();
      // ---- the survivors, in order; rows already in place are not rewritten
      const int P = s_pre;
      const int myrank =
          wbase + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int rk = __shfl(myrank, grp * LPE + bb, 64);
        if (live[bb]) {
          const int rel = P + rk;
          const int64_t dst = off + rel;
          const bool moves = rel != e0 + bb;
          if (moves) {
            const uint32_t ro = (uint32_t)(rel * D + 8 * c) * EB;
            row_store_at<BF16>(kr[bb], Kseg, ro);
            row_store_at<BF16>(vr[bb], Vseg, ro);
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

    // ---- the new entry: after the survivors when compacting
    if (appends) {
      if (!combines) __syncthreads();  // s_u (the combine has a barrier of its own)
      const bool room = len < cap;
      if (room && tid < D) {
        const int64_t dst = (off + npos) * D + tid;
        const float kv = s_tq[G * D + tid];
        if constexpr (BF16) {
          reinterpret_cast<uint16_t*>(a.K)[dst] = f32_to_bf16(kv);     // exact: kv is bf16-rounded
          reinterpret_cast<uint16_t*>(a.V)[dst] = f32_to_bf16(vn[0]);  // exact: a bf16 input
        } else {
          reinterpret_cast<float*>(a.K)[dst] = kv;
          reinterpret_cast<float*>(a.V)[dst] = vn[0];
        }
      }
      if (tid == 0) {
        if (room) {
          a.lam[off + npos] = 0.0f;
          a.lk[off + npos] = s_u[r];
          if (COMPACT && kept) kept[off + npos] = len;
        } else {
          atomicOr(a.status, 1);
        }
        sti_coh(&w.newlen[seg], room ? npos + 1 : npos);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int tile_entries(int d, int nb) { return (64 / (d / 8)) * nb * kDecWaves; }

// Entries per tile (sizes the per-tile workspace rows and flags).
int decode_tile_entries(int d, int g) { return tile_entries(d, decode_nb(d, g)); }

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
  int* newlen = reinterpret_cast<int*>(take(sizeof(int) * S));
  float* part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  float* part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  if (w) {
    w->newlen = newlen;
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

// Compute units of the current device (the persistent grid's size), cached.
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int D, int G, bool BF16>
static hipError_t launch_step(const LayerArgs& a, const DecodeWs& w, const Control& ctl, float tau, bool compact,
                              int32_t* kept, hipStream_t st) {
  const int twg = DecodeShape<D, decode_nb(D, G)>::TWG;
  const int64_t items = (int64_t)a.B + decode_max_tiles(a, twg);
  const int cus = device_cus();
  const int grid = (int)(items < cus ? items : cus);
  if (compact) {
    hipLaunchKernelGGL((decode_step_kernel<D, G, BF16, true>), dim3(grid), dim3(kDecThreads), 0, st, DecodeKArgs{a, w, ctl, tau, kept});
  } else {
    hipLaunchKernelGGL((decode_step_kernel<D, G, BF16, false>), dim3(grid), dim3(kDecThreads), 0, st, DecodeKArgs{a, w, ctl, tau, kept});
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
